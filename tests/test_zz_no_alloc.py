"""GPU check of gdn_prefill_chunked_noalloc (the prefill for callers that cannot
allocate): called through the C ABI, its outputs must equal those of
gdn_prefill_chunked on the same inputs, on two calls in a row, the second
smaller than the first, and must stay within the parity tolerance of the
float64 oracle.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gdn():
    from hybrid_linear_attention_amd import gdn as g
    return g


def rel(x, ref):
    x = x.detach().cpu().double().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def both(gdn, inp, with_h0):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    h0 = d["h0"] if with_h0 else None
    o_ref, ht_ref = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], h0)
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    torch.cuda.synchronize()
    # Python's collector, run during the call, can free device tensors that
    # earlier tests left in reference cycles and lower the count: collect
    # first and keep it off while the count is compared.
    gc.collect()
    gc.disable()
    try:
        before = torch.cuda.memory_allocated()
        gdn.prefill_chunked_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], h0, o=o, ht=ht)
        after = torch.cuda.memory_allocated()
    finally:
        gc.enable()
    torch.cuda.synchronize()
    assert after == before
    return o, ht, o_ref, ht_ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_noalloc_matches_prefill_two_calls(gdn, dtype):
    # first call: the T = 8192 workload (bf16), or the largest fp32 shape the
    # array holds; second call: a smaller ragged batch with an initial state
    T1 = 8192 if dtype == torch.bfloat16 else 64 * 84
    calls = [(synth.prefill_inputs(1, T1, dtype, seed=801), False),
             (synth.prefill_inputs(2, 300, dtype, seed=802, h0_std=0.02), True)]
    for i, (inp, with_h0) in enumerate(calls):
        say("noalloc call", i, dtype, tuple(inp["v"].shape))
        o, ht, o_ref, ht_ref = both(gdn, inp, with_h0)
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
        if i == 1:
            ro, rh = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                    inp["h0"])
            eo, eh = rel(o, ro), rel(ht, rh)
            say("  rel o %.3e ht %.3e" % (eo, eh))
            assert eo <= TOL[dtype] and eh <= TOL[dtype]


def test_noalloc_in_place_state_and_too_large(gdn):
    inp = synth.prefill_inputs(1, 130, torch.bfloat16, seed=803, h0_std=0.02)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o_ref, ht_ref = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"])
    st = d["h0"].clone()
    o = torch.empty_like(o_ref)
    gdn.prefill_chunked_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], st, o=o, ht=st)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(st, ht_ref)
    # beyond the array: rejected before anything is enqueued
    big = torch.empty((1, 64 * 166, 16, 128), dtype=torch.bfloat16, device=DEV)
    bv = torch.empty((1, 64 * 166, 48, 128), dtype=torch.bfloat16, device=DEV)
    ab = torch.empty((1, 64 * 166, 48), dtype=torch.float32, device=DEV)
    with pytest.raises(gdn.GDNError, match="GDN_ERR_TOO_LARGE"):
        gdn.prefill_chunked_noalloc(big, big.clone(), bv, ab, ab.clone(), None,
                                    o=torch.empty_like(bv))
