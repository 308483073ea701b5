"""GPU parity of the gated attention layer (gdn_attn_prefill, gdn_attn_decode)
against the float64 oracle in oracle/attention.py, called through the C ABI.

Tolerances (relative L2 error, float64): 1e-5 for fp32 inputs, 2e-2 for bf16.
Small prefills are compared on every element; the T = 8192 prefill on sampled
query rows of sampled heads (each row attends to its whole prefix), and the
B = 64, 8192-key decode on sampled sequences.
"""
import sys
import time

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A

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
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("B,T", [(1, 1), (1, 37), (2, 64), (1, 200), (2, 321)])
def test_attn_prefill_small(gdn, dtype, B, T):
    say("attn_prefill_small", dtype, B, T)
    inp = synth.attention_inputs(B, T, dtype, seed=100 + T + B)
    d = dev(inp)
    o = gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], d["q_norm_w"], d["k_norm_w"])
    torch.cuda.synchronize()
    ref = A.attention(inp["q"], inp["k"], inp["v"], inp["gate"], inp["q_norm_w"], inp["k_norm_w"])
    e = rel(o, ref)
    say("  rel %.3e" % e)
    assert e <= TOL[dtype]
    assert np.abs(o.cpu().double().numpy() - ref).max() <= 20 * TOL[dtype] * np.abs(ref).max()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_attn_prefill_fills_cache_and_options(gdn, dtype):
    B, T, L = 2, 90, 128
    inp = synth.attention_inputs(B, T, dtype, seed=7)
    d = dev(inp)
    kc = torch.full((B, L, 4, 256), 7.0, dtype=dtype, device=DEV)
    vc = torch.full((B, L, 4, 256), 7.0, dtype=dtype, device=DEV)
    o = gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], d["q_norm_w"], d["k_norm_w"],
                         k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    kref, vref = A.prefill_cache(inp["k"], inp["v"], inp["k_norm_w"])
    assert rel(kc[:, :T], kref) <= TOL[dtype]
    assert torch.equal(vc[:, :T].cpu(), inp["v"])
    assert bool((kc[:, T:] == 7.0).all()) and bool((vc[:, T:] == 7.0).all())
    ref = A.attention(inp["q"], inp["k"], inp["v"], inp["gate"], inp["q_norm_w"], inp["k_norm_w"])
    assert rel(o, ref) <= TOL[dtype]
    # no norm weights, no rotation, another theta
    o2 = gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], rope_dim=0)
    ref2 = A.attention(inp["q"], inp["k"], inp["v"], inp["gate"], rope_dim=0)
    assert rel(o2, ref2) <= TOL[dtype]
    o3 = gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], rope_dim=128, theta=1.0e4)
    ref3 = A.attention(inp["q"], inp["k"], inp["v"], inp["gate"], rope_dim=128, theta=1.0e4)
    assert rel(o3, ref3) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_attn_decode_continues_prefill(gdn, dtype):
    # prefill of 700 tokens into the cache, then 5 decode steps; each step must
    # equal the oracle's decode over the same cache contents
    B, T0, L = 3, 700, 1100
    inp = synth.attention_inputs(B, T0, dtype, seed=21)
    d = dev(inp)
    kc = torch.zeros((B, L, 4, 256), dtype=dtype, device=DEV)
    vc = torch.zeros((B, L, 4, 256), dtype=dtype, device=DEV)
    gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], d["q_norm_w"], d["k_norm_w"],
                     k_cache=kc, v_cache=vc)
    pos_h = np.array([T0, T0 - 200, 3], dtype=np.int32)     # ragged positions per sequence
    for step in range(5):
        s = synth.attention_decode_inputs(B, step, dtype, seed=22)
        sd = dev(s)
        kc_before = kc.cpu()
        vc_before = vc.cpu()
        pos = torch.tensor(pos_h, device=DEV)
        o = gdn.attn_decode(sd["q"], sd["k"], sd["v"], sd["gate"], kc, vc, pos,
                            d["q_norm_w"], d["k_norm_w"])
        torch.cuda.synchronize()
        ref, knew = A.decode(s["q"], s["k"], s["v"], s["gate"], kc_before, vc_before, pos_h,
                             inp["q_norm_w"], inp["k_norm_w"])
        e = rel(o, ref)
        say("  decode step %d rel %.3e" % (step, e))
        assert e <= TOL[dtype]
        for b in range(B):
            assert rel(kc[b, pos_h[b]], knew[b]) <= TOL[dtype]
            assert torch.equal(vc[b, pos_h[b]].cpu(), s["v"][b])
        pos_h = pos_h + 1


def test_attn_prefill_T8192_sampled(gdn):
    T = 8192
    inp = synth.attention_inputs(1, T, torch.bfloat16, seed=1201)
    d = dev(inp)
    t0 = time.time()
    o = gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], d["q_norm_w"], d["k_norm_w"])
    torch.cuda.synchronize()
    say("attn T=8192 on GPU %.1fs" % (time.time() - t0))
    rows = [0, 1, 31, 32, 63, 64, 1000, 4095, 4096, 8000, 8191]
    heads = [0, 5, 6, 17, 23]
    ref = A.attention(inp["q"], inp["k"], inp["v"], inp["gate"], inp["q_norm_w"],
                      inp["k_norm_w"], rows=rows, heads=heads)
    got = o[:, rows][:, :, heads]
    e = rel(got, ref)
    say("attn T=8192 sampled rel %.3e" % e)
    assert e <= 2e-2


def test_attn_decode_B64_8192_sampled(gdn):
    # the decode workload: 64 sequences, 8191 cached keys each (random cache
    # contents stand in for a prefill), one new token at position 8191
    B, L = 64, 8192
    g = torch.Generator().manual_seed(1202)
    kc = torch.randn((B, L, 4, 256), generator=g).to(torch.bfloat16)
    vc = torch.randn((B, L, 4, 256), generator=g).to(torch.bfloat16)
    s = synth.attention_decode_inputs(B, 0, torch.bfloat16, seed=1203)
    kcd, vcd = kc.to(DEV), vc.to(DEV)
    pos_h = np.full(B, L - 1, dtype=np.int32)
    o = gdn.attn_decode(*(s[x].to(DEV) for x in ("q", "k", "v", "gate")), kcd, vcd,
                        torch.tensor(pos_h, device=DEV))
    torch.cuda.synchronize()
    for b in (0, 37, 63):
        ref, _ = A.decode(s["q"][b:b + 1], s["k"][b:b + 1], s["v"][b:b + 1], s["gate"][b:b + 1],
                          kc[b:b + 1], vc[b:b + 1], pos_h[b:b + 1])
        e = rel(o[b:b + 1], ref)
        say("decode b=%d rel %.3e" % (b, e))
        assert e <= 2e-2


def test_attn_deterministic(gdn):
    inp = dev(synth.attention_inputs(1, 300, torch.bfloat16, seed=9))
    o1 = gdn.attn_prefill(inp["q"], inp["k"], inp["v"], inp["gate"])
    o2 = gdn.attn_prefill(inp["q"], inp["k"], inp["v"], inp["gate"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (12, 3), (4, 2)])
def test_attn_other_head_layouts(gdn, dtype, Hq, Hkv):
    # the kernels take the group size Hq / Hkv (1 .. 8) at run time
    say("attn head layout", Hq, Hkv, dtype)
    B, T = 2, 100
    inp = synth.attention_inputs(B, T, dtype, seed=300 + Hq + Hkv, Hq=Hq, Hkv=Hkv)
    d = dev(inp)
    L = 128
    kc = torch.zeros((B, L, Hkv, 256), dtype=dtype, device=DEV)
    vc = torch.zeros((B, L, Hkv, 256), dtype=dtype, device=DEV)
    o = gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], d["q_norm_w"], d["k_norm_w"],
                         k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    ref = A.attention(inp["q"], inp["k"], inp["v"], inp["gate"], inp["q_norm_w"], inp["k_norm_w"])
    assert rel(o, ref) <= TOL[dtype]
    s = synth.attention_decode_inputs(B, 0, dtype, seed=400 + Hq, Hq=Hq, Hkv=Hkv)
    pos_h = np.array([T, T - 37], dtype=np.int32)
    kb, vb = kc.cpu(), vc.cpu()
    od = gdn.attn_decode(*(s[x].to(DEV) for x in ("q", "k", "v", "gate")), kc, vc,
                         torch.tensor(pos_h, device=DEV), d["q_norm_w"], d["k_norm_w"])
    torch.cuda.synchronize()
    refd, _ = A.decode(s["q"], s["k"], s["v"], s["gate"], kb, vb, pos_h, inp["q_norm_w"],
                       inp["k_norm_w"])
    assert rel(od, refd) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_attn_full_rotation_and_first_token(gdn, dtype):
    B, T = 2, 70
    inp = synth.attention_inputs(B, T, dtype, seed=55)
    d = dev(inp)
    # every channel rotates (rope_dim = 256)
    o = gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], d["q_norm_w"], d["k_norm_w"],
                         rope_dim=256, theta=1.0e6)
    torch.cuda.synchronize()
    ref = A.attention(inp["q"], inp["k"], inp["v"], inp["gate"], inp["q_norm_w"],
                      inp["k_norm_w"], rope_dim=256, theta=1.0e6)
    assert rel(o, ref) <= TOL[dtype]
    # decode at position 0 with an empty cache: one key, softmax weight 1, so
    # o = v * sigmoid(gate) for every query head of the group
    L = 64
    kc = torch.zeros((B, L, 4, 256), dtype=dtype, device=DEV)
    vc = torch.zeros((B, L, 4, 256), dtype=dtype, device=DEV)
    s = synth.attention_decode_inputs(B, 3, dtype, seed=56)
    od = gdn.attn_decode(*(s[x].to(DEV) for x in ("q", "k", "v", "gate")), kc, vc,
                         torch.zeros(B, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    v64 = s["v"].double().numpy()
    g64 = s["gate"].double().numpy()
    want = np.stack([v64[:, h // 6] / (1 + np.exp(-g64[:, h])) for h in range(24)], axis=1)
    assert rel(od, want) <= TOL[dtype]
    assert torch.equal(vc[:, 0].cpu(), s["v"])
