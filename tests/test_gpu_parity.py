"""GPU parity: the HIP library, called through its C ABI, against the float64
oracle on the same seeded inputs.

Tolerances (relative L2 error per tensor, e = ||x - ref|| / ||ref||, float64):
* fp32 inputs: 1e-5;  bf16 inputs: 2e-2.

Small cases span several 64-token chunks and a ragged tail and are checked on
every element; the full-size workloads run in the benchmark's launch
configuration and are checked in full (T = 8192 prefill, 64 x 256 decode) or
on sampled value heads that the oracle computes one by one (T = 262,144 and
the packed varlen batch).
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gdn():
    from hybrid_linear_attention_amd import gdn as g
    return g


def rel(x, ref):
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def worst_head(x, ref, axis):
    """Largest relative L2 error over the value heads (entries of ``axis``):
    one head far off cannot hide in the norm of all of them."""
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)
    x, ref = np.moveaxis(x, axis, 0), np.moveaxis(np.asarray(ref, np.float64), axis, 0)
    return max(rel(a, b) for a, b in zip(x, ref))


# one value head of every query/key group (16 groups of 3), at every position
# inside a group
SAMPLED_HEADS = [3 * g + g % 3 for g in range(16)]


def to_dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def run_prefill(gdn, inp, h0=True):
    d = to_dev(inp)
    o, ht = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                d["h0"] if h0 else None)
    torch.cuda.synchronize()
    return o, ht


def oracle_prefill(inp, h0=True):
    return oracle.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                          inp["h0"] if h0 else None)


# ------------------------------------------------------------------ small prefill
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("B,T,h0std", [(1, 64, 0.0), (1, 200, 0.02), (2, 130, 0.02),
                                       (1, 1, 0.02), (3, 63, 0.0), (1, 321, 0.5)])
def test_prefill_small(gdn, dtype, B, T, h0std):
    say("prefill_small", dtype, B, T, h0std)
    inp = synth.prefill_inputs(B, T, dtype, seed=7 + T + B, h0_std=h0std)
    o, ht = run_prefill(gdn, inp)
    o_ref, ht_ref = oracle_prefill(inp)
    eo, eh = worst_head(o, o_ref, 2), worst_head(ht, ht_ref, 1)
    say("  worst head rel o %.3e ht %.3e" % (eo, eh))
    assert eo <= TOL[dtype] and eh <= TOL[dtype]
    # element-wise, per head: no single output far off (guards against a
    # masked-row bug hiding in the norm)
    on = o.cpu().double().numpy()
    err = max(np.abs(on[:, :, h] - o_ref[:, :, h]).max() / np.abs(o_ref[:, :, h]).max()
              for h in range(on.shape[2]))
    say("  worst head max element error / max |o| %.3e" % err)
    assert err <= 5 * TOL[dtype]


def test_prefill_T0_passes_state(gdn):
    inp = synth.prefill_inputs(2, 0, torch.bfloat16, seed=3, h0_std=0.1)
    o, ht = run_prefill(gdn, inp)
    assert o.shape == (2, 0, 48, 128)
    assert torch.equal(ht.cpu(), inp["h0"])


def test_prefill_without_h0_and_without_ht(gdn):
    inp = synth.prefill_inputs(1, 100, torch.bfloat16, seed=4)
    d = to_dev(inp)
    o, ht = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None,
                                output_final_state=False)
    torch.cuda.synchronize()
    assert ht is None
    o_ref, _ = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], None)
    assert rel(o, o_ref) <= 2e-2


def test_prepare_then_scan_equals_chunked(gdn):
    inp = to_dev(synth.prefill_inputs(1, 300, torch.bfloat16, seed=5, h0_std=0.02))
    o1, ht1 = gdn.prefill_chunked(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["h0"])
    o2 = torch.empty_like(o1)
    ht2 = torch.empty_like(ht1)
    ws = torch.empty(gdn.prefill_workspace_bytes(1, 300, 16, 48), dtype=torch.uint8, device=DEV)
    gdn.prefill_prepare(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["h0"], o2, ht2, ws)
    gdn.prefill_scan(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["h0"], o2, ht2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)


def test_prefill_deterministic(gdn):
    inp = synth.prefill_inputs(1, 500, torch.bfloat16, seed=6, h0_std=0.02)
    o1, ht1 = run_prefill(gdn, inp)
    o2, ht2 = run_prefill(gdn, inp)
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)


def test_prefill_in_place_carry_and_split(gdn):
    """ht may be exactly h0; two calls with the state carried equal one call."""
    T1, T2 = 130, 77
    inp = synth.prefill_inputs(1, T1 + T2, torch.bfloat16, seed=8, h0_std=0.02)
    d = to_dev(inp)
    o_all, ht_all = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"])
    st = d["h0"].clone()
    sl1 = [x[:, :T1].contiguous() for x in (d["q"], d["k"], d["v"], d["alpha"], d["beta"])]
    sl2 = [x[:, T1:].contiguous() for x in (d["q"], d["k"], d["v"], d["alpha"], d["beta"])]
    o1, _ = gdn.prefill_chunked(*sl1, st, ht=st)
    o2, _ = gdn.prefill_chunked(*sl2, st, ht=st)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle_prefill(inp)
    assert rel(torch.cat([o1, o2], 1), o_ref) <= 2e-2
    assert rel(st, ht_ref) <= 2e-2
    assert rel(o_all, o_ref) <= 2e-2 and rel(ht_all, ht_ref) <= 2e-2


def test_prefill_identity_invariant_fp32(gdn):
    """beta = 0, alpha = 1: the state is untouched and o_t = S0 q_t."""
    inp = synth.prefill_inputs(1, 150, torch.float32, seed=9, h0_std=0.3)
    inp["beta"].zero_()
    inp["alpha"].fill_(1.0)
    o, ht = run_prefill(gdn, inp)
    assert rel(ht, inp["h0"].double().numpy()) <= 1e-6
    S0 = inp["h0"][0].double()
    qh = inp["q"][0].double()[:, torch.arange(48) // 3]           # [T,48,D]
    ref = torch.einsum("hij,thj->thi", S0, qh)
    assert rel(o[0], ref.numpy()) <= 1e-5


def test_prefill_orthonormal_retrieval_fp32(gdn):
    """alpha = beta = 1, orthonormal keys, S0 = 0: querying with k_t returns v_t."""
    T = 128
    g = torch.Generator().manual_seed(11)
    keys = []
    for _ in range(16):
        Qm, _ = torch.linalg.qr(torch.randn(128, 128, generator=g, dtype=torch.float64))
        keys.append(Qm.T[:T])
    k = torch.stack(keys, 1)[None].float().contiguous()           # [1,T,16,128]
    v = torch.randn(1, T, 48, 128, generator=g).contiguous()
    ones = torch.ones(1, T, 48)
    inp = dict(q=k.clone(), k=k, v=v, alpha=ones.clone(), beta=ones.clone(), h0=None)
    o, ht = run_prefill(gdn, inp, h0=False)
    assert rel(o, v.double().numpy()) <= 1e-5


def test_head_map_contiguous_groups(gdn):
    """Value head h reads query/key head h // 3: permuting query/key heads
    permutes exactly the matching value-head groups."""
    inp = synth.prefill_inputs(1, 96, torch.float32, seed=12, h0_std=0.0)
    o, _ = run_prefill(gdn, inp, h0=False)
    perm = torch.tensor([1, 0] + list(range(2, 16)))
    inp2 = dict(inp)
    inp2["q"] = inp["q"][:, :, perm].contiguous()
    inp2["k"] = inp["k"][:, :, perm].contiguous()
    vperm = torch.cat([torch.arange(3, 6), torch.arange(0, 3), torch.arange(6, 48)])
    inp2["v"] = inp["v"][:, :, vperm].contiguous()
    inp2["alpha"] = inp["alpha"][:, :, vperm].contiguous()
    inp2["beta"] = inp["beta"][:, :, vperm].contiguous()
    o2, _ = run_prefill(gdn, inp2, h0=False)
    assert torch.allclose(o2[:, :, vperm], o, rtol=0, atol=1e-6)


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_decode_small(gdn, dtype):
    B, steps = 5, 6
    say("decode_small", dtype)
    st = synth.decode_state(B, seed=21, std=0.05).to(DEV)
    ref = st.cpu().double().numpy().copy()
    worst = 0.0
    for s in range(steps):
        d = synth.decode_step_inputs(B, s, dtype, seed=21)
        dd = to_dev(d)
        o = gdn.decode_step(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], st)
        o_ref, ref = oracle.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref,
                                         inplace=True)
        torch.cuda.synchronize()
        worst = max(worst, rel(o, o_ref))
    worst = max(worst, rel(st, ref))
    say("  worst rel %.3e" % worst)
    assert worst <= TOL[dtype]


def test_decode_steps_equal_fp32_prefill(gdn):
    """256 fp32 decode steps reach the fp32 chunked prefill of the same tokens."""
    T = 256
    inp = synth.prefill_inputs(1, T, torch.float32, seed=22, h0_std=0.02)
    o_p, ht_p = run_prefill(gdn, inp)
    d = to_dev(inp)
    st = d["h0"].clone()
    outs = []
    for t in range(T):
        outs.append(gdn.decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                    d["v"][:, t].contiguous(), d["alpha"][:, t].contiguous(),
                                    d["beta"][:, t].contiguous(), st))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, 1)
    assert rel(o_d, o_p.cpu().double().numpy()) <= 1e-5
    assert rel(st, ht_p.cpu().double().numpy()) <= 1e-5


# ------------------------------------------------------------------ bf16 state storage
def _bf16(x64):
    """float64 array holding bfloat16 values -> bfloat16 tensor (exact)."""
    return torch.from_numpy(np.asarray(x64, dtype=np.float64)).float().to(torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_decode_bf16_state_small(gdn, dtype):
    B, steps = 5, 6
    say("decode_bf16_state_small", dtype)
    st = synth.decode_state(B, seed=31, std=0.05).to(torch.bfloat16).to(DEV)
    ref = st.cpu().double().numpy().copy()
    worst = 0.0
    for s in range(steps):
        d = synth.decode_step_inputs(B, s, dtype, seed=31)
        dd = to_dev(d)
        o = gdn.decode_step(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], st)
        o_ref, ref = oracle.decode_step_bf16_state(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                                   ref)
        torch.cuda.synchronize()
        worst = max(worst, rel(o, o_ref))
    worst = max(worst, rel(st, ref))
    say("  worst rel %.3e" % worst)
    assert st.dtype == torch.bfloat16 and worst <= 2e-2


def test_decode_bf16_state_64x64(gdn):
    """The decode workload's batch (64 sequences) with the state in bf16, for
    64 steps (each oracle step rounds 50 M state elements on the host)."""
    B, steps = 64, 64
    st = synth.decode_state(B, 1002, 0.02).to(torch.bfloat16)
    ref = st.double().numpy().copy()
    st = st.to(DEV)
    worst = 0.0
    t0 = time.time()
    for s in range(steps):
        d = synth.decode_step_inputs(B, s, torch.bfloat16, seed=1002)
        dd = to_dev(d)
        o = gdn.decode_step(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], st)
        o_ref, ref = oracle.decode_step_bf16_state(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                                   ref)
        worst = max(worst, rel(o, o_ref))
        if s % 16 == 0:
            say("  bf16-state decode step %d worst %.3e (%.1fs)" % (s, worst, time.time() - t0))
    worst = max(worst, rel(st, ref))
    say("decode bf16 state 64x64 worst rel %.3e" % worst)
    assert worst <= 2e-2


@pytest.mark.parametrize("T", [0, 64, 150], ids=["T0", "T64", "T150"])
def test_prefill_bf16_state(gdn, T):
    inp = synth.prefill_inputs(2, T, torch.bfloat16, seed=33, h0_std=0.05)
    h0 = inp["h0"].to(torch.bfloat16)
    d = to_dev(inp)
    o, ht = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], h0.to(DEV))
    torch.cuda.synchronize()
    assert ht.dtype == torch.bfloat16
    if T == 0:
        assert torch.equal(ht.cpu(), h0)                 # passes the state through exactly
        return
    o_ref, ht_ref = oracle.prefill_bf16_state(inp["q"], inp["k"], inp["v"], inp["alpha"],
                                              inp["beta"], h0)
    eo, eh = rel(o, o_ref), rel(ht, ht_ref)
    say("prefill bf16 state T=%d rel o %.3e ht %.3e" % (T, eo, eh))
    assert eo <= 2e-2 and eh <= 2e-2
    # the same call with the final state written over h0
    hin = h0.to(DEV)
    o2, ht2 = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], hin, ht=hin)
    torch.cuda.synchronize()
    assert ht2.data_ptr() == hin.data_ptr()
    assert torch.equal(o2, o) and torch.equal(ht2, ht)


def test_bf16_state_prefill_then_decode(gdn):
    """Carry in bf16: a prefill's final state continues in decode steps."""
    T, steps = 130, 8
    inp = synth.prefill_inputs(1, T, torch.bfloat16, seed=34, h0_std=0.02)
    h0 = inp["h0"].to(torch.bfloat16)
    d = to_dev(inp)
    _, st = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], h0.to(DEV))
    _, ref = oracle.prefill_bf16_state(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], h0)
    worst = rel(st, ref)
    for s in range(steps):
        dd = synth.decode_step_inputs(1, s, torch.bfloat16, seed=34)
        o = gdn.decode_step(*(dd[x].to(DEV) for x in ("q", "k", "v", "alpha", "beta")), st)
        o_ref, ref = oracle.decode_step_bf16_state(dd["q"], dd["k"], dd["v"], dd["alpha"],
                                                   dd["beta"], ref)
        worst = max(worst, rel(o, o_ref))
    worst = max(worst, rel(st, ref))
    say("bf16 carry prefill -> decode worst rel %.3e" % worst)
    assert worst <= 2e-2


# ------------------------------------------------------------------ speculative decoding
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_verify_commit_small(gdn, dtype):
    B, n = 6, 3
    d = synth.prefill_inputs(B, n, dtype, seed=41)
    st = synth.decode_state(B, seed=41, std=0.05)
    dd = to_dev(d)
    sd = st.to(DEV)
    o = gdn.decode_verify(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], sd)
    torch.cuda.synchronize()
    assert torch.equal(sd.cpu(), st)                  # verify leaves the state alone
    o_ref = oracle.decode_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], st)
    eo = rel(o, o_ref)
    acc = torch.tensor([0, 1, 2, 3, 7, -2], dtype=torch.int32)   # 7 and -2 are clamped
    gdn.decode_commit(dd["k"], dd["v"], dd["alpha"], dd["beta"], sd, acc.to(DEV))
    torch.cuda.synchronize()
    s_ref = oracle.decode_commit(d["k"], d["v"], d["alpha"], d["beta"], st, acc.numpy())
    es = rel(sd, s_ref)
    assert torch.equal(sd[0].cpu(), st[0]) and torch.equal(sd[5].cpu(), st[5])
    # after committing m tokens, verifying the rest reproduces the first verify
    m = 1
    s1 = st.to(DEV)
    gdn.decode_commit(dd["k"], dd["v"], dd["alpha"], dd["beta"], s1,
                      torch.full((B,), m, dtype=torch.int32, device=DEV))
    rest = {x: dd[x][:, m:].contiguous() for x in ("q", "k", "v", "alpha", "beta")}
    o2 = gdn.decode_verify(rest["q"], rest["k"], rest["v"], rest["alpha"], rest["beta"], s1)
    torch.cuda.synchronize()
    ec = rel(o2, o[:, m:].cpu().double().numpy())
    say("verify/commit %s rel o %.3e state %.3e consistency %.3e" % (dtype, eo, es, ec))
    tol = TOL[dtype]
    assert eo <= tol and es <= tol and ec <= tol


def test_verify_commit_rounds(gdn):
    """64 sequences, drafts of 3 tokens (two MTP drafts plus the next token),
    16 rounds of verify + commit with seeded acceptance counts."""
    B, n, rounds = 64, 3, 16
    st = synth.decode_state(B, 1002, 0.02)
    ref = st.double().numpy().copy()
    sd = st.to(DEV)
    gen = torch.Generator().manual_seed(4242)
    worst = 0.0
    for rd in range(rounds):
        d = synth.prefill_inputs(B, n, torch.bfloat16, seed=5000 + rd)
        dd = to_dev(d)
        o = gdn.decode_verify(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], sd)
        acc = torch.randint(0, n + 1, (B,), generator=gen, dtype=torch.int32)
        gdn.decode_commit(dd["k"], dd["v"], dd["alpha"], dd["beta"], sd, acc.to(DEV))
        o_ref = oracle.decode_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref)
        ref = oracle.decode_commit(d["k"], d["v"], d["alpha"], d["beta"], ref, acc.numpy())
        worst = max(worst, rel(o, o_ref))
    worst = max(worst, rel(sd, ref))
    say("verify/commit 64 x 16 rounds worst rel %.3e" % worst)
    assert worst <= 2e-2


# ------------------------------------------------------------------ varlen
@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_varlen_small(gdn, dtype, gated):
    lengths = [1, 64, 0, 130, 65, 257]
    say("varlen_small", dtype, gated)
    inp = synth.varlen_inputs(lengths, dtype=dtype, seed=31, h0_std=0.05, gate=gated)
    d = to_dev(inp)
    w = torch.linspace(0.5, 1.5, 128)
    y, ht = gdn.prefill_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                               d["h0"], gate=d["gate"], norm_weight=w.to(DEV) if gated else None,
                               norm_eps=1e-6)
    torch.cuda.synchronize()
    y_ref, ht_ref = oracle.varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  inp["cu_seqlens"].numpy(), inp["h0"], gate=inp["gate"],
                                  norm_weight=w.numpy() if gated else None, eps=1e-6)
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lengths)):
        s, e = cu[n], cu[n + 1]
        if e > s:
            assert rel(y[s:e], y_ref[s:e]) <= TOL[dtype], n
        assert rel(ht[n], ht_ref[n]) <= TOL[dtype], n
    assert torch.equal(ht[2].cpu(), inp["h0"][2])          # empty sequence


def test_varlen_equals_separate_calls(gdn):
    lengths = [100, 7, 200]
    inp = to_dev(synth.varlen_inputs(lengths, dtype=torch.bfloat16, seed=32, h0_std=0.02, gate=False))
    y, ht = gdn.prefill_varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                               inp["cu_seqlens"], inp["h0"])
    cu = inp["cu_seqlens"].tolist()
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        o_n, ht_n = gdn.prefill_chunked(*(x[None, s:e].contiguous() for x in
                                          (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])),
                                        inp["h0"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o_n[0], y[s:e])
        assert torch.equal(ht_n[0], ht[n])


# ------------------------------------------------------------------ head-wide scan
# bf16 calls with at least 128 (sequence, value head) pairs run the head-wide
# scan (one workgroup per head and sequence, gated epilogue inside); smaller
# calls run the split scan (and a separate gated pass).  Both perform the same
# products in the same order, so their plain outputs agree bit for bit.

def test_head_scan_equals_split_scan_bitwise(gdn):
    lengths = [200, 64, 1, 333, 129, 70]                   # 6 x 48 = 288 pairs: head-wide
    inp = synth.varlen_inputs(lengths, dtype=torch.bfloat16, seed=91, h0_std=0.05, gate=False)
    d = to_dev(inp)
    o, ht = gdn.prefill_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                               d["h0"])
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lengths)):                          # 48 pairs each: split scan
        s, e = cu[n], cu[n + 1]
        o_n, ht_n = gdn.prefill_chunked(*(x[None, s:e].contiguous() for x in
                                          (d["q"], d["k"], d["v"], d["alpha"], d["beta"])),
                                        d["h0"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o_n[0], o[s:e]), n
        assert torch.equal(ht_n[0], ht[n]), n


@pytest.mark.parametrize("B,T,Hqk,Hv", [(6, 150, 16, 48), (4, 100, 4, 64), (3, 70, 32, 96),
                                         (2, 90, 16, 64)])     # 128 pairs: the threshold
def test_head_scan_against_oracle(gdn, B, T, Hqk, Hv):
    say("head scan", B, T, Hqk, Hv)
    inp = synth.prefill_inputs(B, T, torch.bfloat16, seed=92 + T, h0_std=0.05, Hqk=Hqk, Hv=Hv)
    o, ht = run_prefill(gdn, inp)
    o_ref, ht_ref = oracle_prefill(inp)
    eo, eh = worst_head(o, o_ref, 2), worst_head(ht, ht_ref, 1)
    say("  worst head rel o %.3e ht %.3e" % (eo, eh))
    assert eo <= 2e-2 and eh <= 2e-2


# one sequence (48 pairs): split scan + the separate gated pass; six
# sequences (288 pairs): the head-wide scan with the epilogue inside
@pytest.mark.parametrize("lengths", [[300], [64, 1, 130, 0, 77, 200]])
def test_head_scan_gated_strong_decay(gdn, lengths):
    inp = synth.varlen_inputs(lengths, dtype=torch.bfloat16, seed=93, h0_std=0.05, gate=True,
                              strong_decay=True)
    d = to_dev(inp)
    w = torch.linspace(1.5, 0.5, 128)
    y, ht = gdn.prefill_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                               d["h0"], gate=d["gate"], norm_weight=w.to(DEV), norm_eps=1e-6)
    torch.cuda.synchronize()
    y_ref, ht_ref = oracle.varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  inp["cu_seqlens"].numpy(), inp["h0"], gate=inp["gate"],
                                  norm_weight=w.numpy(), eps=1e-6)
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lengths)):
        s, e = cu[n], cu[n + 1]
        if e > s:
            ey = worst_head(y[s:e], y_ref[s:e], 1)
            say("  gated seq %d worst head rel %.3e" % (n, ey))
            assert ey <= 2e-2, n
        assert worst_head(ht[n], ht_ref[n], 0) <= 2e-2, n


# ------------------------------------------------------------------ full-size workloads
def test_config0_T256_fp32(gdn):
    c = synth.CONFIGS[0]
    inp = synth.config_inputs(0)
    o, ht = run_prefill(gdn, inp, h0=False)
    o_ref, ht_ref = oracle_prefill(inp, h0=False)
    eo, eh = worst_head(o, o_ref, 2), worst_head(ht, ht_ref, 1)
    say("config0 worst head rel o %.3e ht %.3e (all heads %.3e %.3e)"
        % (eo, eh, rel(o, o_ref), rel(ht, ht_ref)))
    assert eo <= 1e-5 and eh <= 1e-5 and c["dtype"] == torch.float32


def test_config1_T8192_bf16(gdn):
    inp = synth.config_inputs(1)
    t0 = time.time()
    o, ht = run_prefill(gdn, inp, h0=False)
    o_ref, ht_ref = oracle_prefill(inp, h0=False)
    eo, eh = worst_head(o, o_ref, 2), worst_head(ht, ht_ref, 1)
    say("config1 worst head rel o %.3e ht %.3e (all heads %.3e %.3e, %.1fs)"
        % (eo, eh, rel(o, o_ref), rel(ht, ht_ref), time.time() - t0))
    assert eo <= 2e-2 and eh <= 2e-2


def test_config2_decode_64x256_bf16(gdn):
    c = synth.CONFIGS[2]
    B, steps = c["B"], c["steps"]
    st = synth.decode_state(B, c["seed"], c["h0_std"])
    ref = st.double().numpy().copy()
    st = st.to(DEV)
    worst = 0.0
    t0 = time.time()
    for s in range(steps):
        d = synth.decode_step_inputs(B, s, c["dtype"], seed=c["seed"])
        dd = to_dev(d)
        o = gdn.decode_step(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], st)
        o_ref, ref = oracle.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref,
                                         inplace=True)
        worst = max(worst, rel(o, o_ref))
        if s % 64 == 0:
            say("  decode step %d worst %.3e (%.1fs)" % (s, worst, time.time() - t0))
    worst = max(worst, rel(st, ref))
    say("config2 worst rel %.3e" % worst)
    assert worst <= 2e-2


def test_config3_T262144_sampled_heads(gdn):
    c = synth.CONFIGS[3]
    inp = synth.config_inputs(3)
    say("config3 inputs ready")
    o, ht = run_prefill(gdn, inp)
    heads = SAMPLED_HEADS
    sub = oracle.subset_heads(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                              inp["h0"], heads, 16, 48)
    t0 = time.time()
    o_ref, ht_ref = oracle.prefill(*sub)
    say("config3 oracle %.1fs" % (time.time() - t0))
    for i, h in enumerate(heads):
        eo, eh = rel(o[0, :, h], o_ref[0, :, i]), rel(ht[0, h], ht_ref[0, i])
        say("config3 head %d rel o %.3e ht %.3e" % (h, eo, eh))
        assert eo <= 2e-2 and eh <= 2e-2
    assert c["T"] == 262144


def test_config4_varlen_sampled_heads(gdn):
    c = synth.CONFIGS[4]
    inp = synth.config_inputs(4)
    say("config4 lengths", inp["lengths"])
    d = to_dev(inp)
    y, ht = gdn.prefill_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                               d["h0"], gate=d["gate"], norm_eps=1e-6)
    torch.cuda.synchronize()
    heads = SAMPLED_HEADS
    q_s, k_s, v_s, a_s, b_s, h_s = oracle.subset_heads(inp["q"], inp["k"], inp["v"],
                                                       inp["alpha"], inp["beta"], inp["h0"],
                                                       heads, 16, 48)
    gate_s = inp["gate"][:, heads]
    t0 = time.time()
    y_ref, ht_ref = oracle.varlen(q_s, k_s, v_s, a_s, b_s, inp["cu_seqlens"].numpy(), h_s,
                                  gate=gate_s, eps=1e-6)
    say("config4 oracle %.1fs" % (time.time() - t0))
    cu = inp["cu_seqlens"].tolist()
    for n in range(c["N"]):
        s, e = cu[n], cu[n + 1]
        for i, h in enumerate(heads):
            ey = rel(y[s:e, h], y_ref[s:e, i])
            eh = rel(ht[n, h], ht_ref[n, i])
            assert ey <= 2e-2 and eh <= 2e-2, (n, h, ey, eh)
    say("config4 ok")


# ------------------------------------------------------------------ backward
GRAD_NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dh0")


def run_backward(gdn, inp):
    d = to_dev(inp)
    g = gdn.prefill_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["do"],
                             d["h0"], d["dht"])
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("B,T,h0std,dhtstd", [(1, 64, 0.0, 0.0), (1, 200, 0.02, 0.02),
                                              (2, 130, 0.02, 0.0), (1, 1, 0.02, 0.02),
                                              (3, 63, 0.0, 0.02), (1, 321, 0.5, 0.1)])
def test_backward_small(gdn, dtype, B, T, h0std, dhtstd):
    say("backward_small", dtype, B, T, h0std, dhtstd)
    inp = synth.backward_inputs(B, T, dtype, seed=11 + T + B, h0_std=h0std, dht_std=dhtstd)
    got = run_backward(gdn, inp)
    ref = oracle.prefill_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  inp["do"], inp["h0"], inp["dht"])
    errs = [rel(x, y) for x, y in zip(got, ref)]
    say("  rel " + " ".join("%s %.3e" % (n, e) for n, e in zip(GRAD_NAMES, errs)))
    for n, e in zip(GRAD_NAMES, errs):
        assert e <= TOL[dtype], (n, e)


def test_backward_T0(gdn):
    inp = synth.backward_inputs(2, 0, torch.bfloat16, seed=5, h0_std=0.1, dht_std=0.1)
    got = run_backward(gdn, inp)
    assert got[0].shape == (2, 0, 16, 128)
    assert torch.equal(got[5].cpu(), inp["dht"])
    inp["dht"] = None
    got = run_backward(gdn, inp)
    assert torch.count_nonzero(got[5]).item() == 0


def test_backward_deterministic(gdn):
    inp = synth.backward_inputs(1, 300, torch.bfloat16, seed=9, h0_std=0.02, dht_std=0.02)
    g1 = run_backward(gdn, inp)
    g2 = run_backward(gdn, inp)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_T8192_sampled_groups(gdn):
    # the training shape of the prefill workload: whole call on the GPU, two
    # query/key groups (their three value heads each) checked against the oracle
    inp = synth.backward_inputs(1, 8192, torch.bfloat16, seed=1011, h0_std=0.02,
                                dht_std=0.02)
    got = run_backward(gdn, inp)
    say("backward T=8192 done on GPU")
    for gq in (0, 15):
        heads = [3 * gq, 3 * gq + 1, 3 * gq + 2]
        sub = oracle.subset_heads(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  inp["h0"], heads, 16, 48)
        do_s = inp["do"][:, :, heads]
        dht_s = inp["dht"][:, heads]
        t0 = time.time()
        # one query/key head shared by the three value heads, as in the call
        ref = oracle.prefill_backward(sub[0][:, :, :1], sub[1][:, :, :1], sub[2], sub[3],
                                      sub[4], do_s, sub[5], dht_s)
        say("  oracle group %d %.1fs" % (gq, time.time() - t0))
        mine = (got[0][:, :, gq:gq + 1], got[1][:, :, gq:gq + 1], got[2][:, :, heads],
                got[3][:, :, heads], got[4][:, :, heads], got[5][:, heads])
        errs = [rel(x, y) for x, y in zip(mine, ref)]
        say("  group %d rel " % gq + " ".join("%s %.3e" % (n, e) for n, e in zip(GRAD_NAMES, errs)))
        for n, e in zip(GRAD_NAMES, errs):
            assert e <= 2e-2, (gq, n, e)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("Hqk,Hv", [(8, 8), (4, 16)])
def test_backward_other_head_layouts(gdn, dtype, Hqk, Hv):
    # the gradient kernel walks the Hv / Hqk value heads of a group at run time
    say("backward head layout", Hqk, Hv, dtype)
    inp = synth.backward_inputs(1, 150, dtype, seed=61 + Hv, h0_std=0.02, dht_std=0.02,
                                Hqk=Hqk, Hv=Hv)
    got = run_backward(gdn, inp)
    ref = oracle.prefill_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  inp["do"], inp["h0"], inp["dht"])
    for n, x, y in zip(GRAD_NAMES, got, ref):
        e = rel(x, y)
        assert e <= TOL[dtype], (n, e)


def test_autograd_function_matches_oracle(gdn):
    # the differentiable wrapper: forward and backward through the library,
    # gradients of sum(o * do) + sum(ht * dht) against the float64 oracle
    inp = synth.backward_inputs(1, 130, torch.bfloat16, seed=71, h0_std=0.02, dht_std=0.02)
    d = {k: (v.to(DEV).requires_grad_(k not in ("do", "dht")) if v is not None else None)
         for k, v in inp.items()}
    o, ht = gdn.gated_delta_rule(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"])
    loss = (o.float() * d["do"].float()).sum() + (ht * d["dht"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    ref = oracle.prefill_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  inp["do"], inp["h0"], inp["dht"])
    for name, key, r in zip(GRAD_NAMES, ("q", "k", "v", "alpha", "beta", "h0"), ref):
        e = rel(d[key].grad, r)
        assert e <= 2e-2, (name, e)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_varlen_backward_equals_separate_sequences(gdn, dtype):
    # packed backward vs the oracle's backward of each sequence on its own,
    # with a zero-length and a one-token sequence in the batch
    lengths = [70, 0, 129, 64, 1]
    vl = synth.varlen_inputs(lengths, dtype=dtype, seed=83, h0_std=0.02, gate=False)
    gen = torch.Generator().manual_seed(84)
    T_tot, N = sum(lengths), len(lengths)
    do = torch.randn((T_tot, 48, 128), generator=gen).to(dtype)
    dht = torch.randn((N, 48, 128, 128), generator=gen) * 0.02
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in vl.items()}
    got = gdn.prefill_varlen_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                      d["cu_seqlens"], do.to(DEV), d["h0"], dht.to(DEV))
    torch.cuda.synchronize()
    cu = vl["cu_seqlens"].tolist()
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        sl = lambda x: x[s:e][None]
        ref = oracle.prefill_backward(sl(vl["q"]), sl(vl["k"]), sl(vl["v"]), sl(vl["alpha"]),
                                      sl(vl["beta"]), sl(do), vl["h0"][n:n + 1], dht[n:n + 1])
        mine = (got[0][s:e], got[1][s:e], got[2][s:e], got[3][s:e], got[4][s:e], got[5][n])
        for name, x, y in zip(GRAD_NAMES, mine, ref):
            y = y[0]
            if y.size == 0:
                continue
            err = rel(x, y)
            assert err <= TOL[dtype], (n, name, err)


def test_graph_capture_replays_match_eager(gdn):
    # every entry point only enqueues work on the current stream, so a HIP
    # graph can hold them: four decode steps and a chunked prefill, replayed
    # three times with eager work in between, each replay checked bitwise
    # against the same calls run eagerly
    B = 8
    st0 = synth.decode_state(B, 91, 0.02).to(DEV)
    steps = [to_dev(synth.decode_step_inputs(B, s, torch.bfloat16, seed=92)) for s in range(4)]
    pre = to_dev(synth.prefill_inputs(1, 200, torch.bfloat16, seed=93, h0_std=0.02))
    ws = torch.empty(gdn.prefill_workspace_bytes(1, 200, 16, 48), dtype=torch.uint8, device=DEV)
    outs = [torch.empty((B, 48, 128), dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    o_pre = torch.empty((1, 200, 48, 128), dtype=torch.bfloat16, device=DEV)
    ht_pre = torch.empty((1, 48, 128, 128), dtype=torch.float32, device=DEV)
    state = st0.clone()

    def work():
        for s, d in enumerate(steps):
            gdn.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], state, o=outs[s])
        gdn.prefill_chunked(pre["q"], pre["k"], pre["v"], pre["alpha"], pre["beta"], pre["h0"],
                            o=o_pre, ht=ht_pre, workspace=ws)

    work()                                   # eager reference
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs] + [state.clone(), o_pre.clone(), ht_pre.clone()]
    state.copy_(st0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.synchronize()
    for rep in range(3):
        state.copy_(st0)                     # eager work between replays
        for x in outs:
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outs + [state, o_pre, ht_pre]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep


def test_debug_mode_rejects_malformed_cu_seqlens(gdn, monkeypatch):
    # GDN_DEBUG=1: the packed calls read cu_seqlens on the host and refuse
    # offsets that decrease or do not end at T_tot; without it they never read
    vl = synth.varlen_inputs([40, 60], dtype=torch.bfloat16, seed=95, gate=False)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in vl.items()}
    monkeypatch.setenv("GDN_DEBUG", "1")
    y, _ = gdn.prefill_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                              d["h0"])
    torch.cuda.synchronize()
    for bad in ([0, 70, 60], [0, 40, 99], [5, 40, 100]):
        cu = torch.tensor(bad, dtype=torch.int32, device=DEV)
        with pytest.raises(gdn.GDNError) as ei:
            gdn.prefill_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], cu, d["h0"])
        assert ei.value.status == -2
        do = torch.zeros((100, 48, 128), dtype=torch.bfloat16, device=DEV)
        with pytest.raises(gdn.GDNError) as ei:
            gdn.prefill_varlen_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], cu, do)
        assert ei.value.status == -2
