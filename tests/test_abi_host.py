"""Host-only checks of the C ABI: the library loads, exports every entry point
include/gdn.h declares, sizes workspaces as documented, and rejects bad
arguments with the documented status code before anything is enqueued.

Every call here fails validation on purpose (fake, never-dereferenced device
addresses), so no kernel is launched and no GPU is needed.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EALIAS, EWS, EHIP = 0, -1, -2, -3, -4, -5, -6, -7
ETOOLARGE = -8
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def gdn():
    from hybrid_linear_attention_amd import gdn as g
    return g


@pytest.fixture(scope="module")
def lib(gdn):
    return gdn.lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("gdn_prefill_chunked", "gdn_decode_step", "gdn_prefill_varlen"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(gdn):
    for code in (OK, ENULL, ESHAPE, EUNSUP, EALIGN, EALIAS, EWS, EHIP, ETOOLARGE):
        s = gdn.status_str(code)
        assert s.startswith("GDN_")
    assert "unknown" in gdn.status_str(12345)
    assert gdn.abi_version() == 100


def test_workspace_sizes(gdn):
    # per chunk: Tt and M (48 x 64 x 64 elements each), gam and dec (48 x 64
    # fp32 each)
    per_chunk_bf16 = 2 * 48 * 4096 * 2 + 2 * 48 * 64 * 4
    assert gdn.prefill_workspace_bytes(1, 0, 16, 48) == 0
    w1 = gdn.prefill_workspace_bytes(1, 64, 16, 48)
    w2 = gdn.prefill_workspace_bytes(1, 128, 16, 48)
    w3 = gdn.prefill_workspace_bytes(1, 65, 16, 48)
    assert w2 - w1 == per_chunk_bf16
    assert w3 == w2                       # a ragged tail is one more chunk
    assert gdn.prefill_workspace_bytes(2, 64, 16, 48) == w2
    w32 = gdn.prefill_workspace_bytes(1, 64, 16, 48, dtype=__import__("torch").float32)
    assert w32 > w1
    # the state never lives in the workspace: nothing in it scales with D*D per head
    assert w1 < 48 * 128 * 128 * 4
    assert gdn.prefill_workspace_bytes(1, 64, 16, 48, D=64) == 0
    assert gdn.prefill_workspace_bytes(1, 64, 16, 47) == 0
    # varlen: ceil(T_tot/64) + N chunks plus the chunk table
    assert gdn.varlen_workspace_bytes(3, 100, 16, 48) >= gdn.prefill_workspace_bytes(1, 64 * 5, 16, 48)


# fake device addresses, 256-byte aligned and far apart (never dereferenced)
BASE = 0x7F0000000000
STRIDE = 1 << 36


def addr(i, off=0):
    return ctypes.c_void_p(BASE + i * STRIDE + off)


def prefill_call(lib, name="gdn_prefill_chunked", **kw):
    args = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), h0=addr(5),
                o=addr(6), ht=addr(7), B=1, T=128, Hqk=16, Hv=48, D=128, dt=BF16,
                ws=addr(8), ws_bytes=1 << 40, stream=None)
    args.update(kw)
    fn = getattr(lib, name)
    return fn(args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["h0"],
              args["o"], args["ht"], args["B"], args["T"], args["Hqk"], args["Hv"], args["D"],
              args["dt"], args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("name", ["gdn_prefill_chunked", "gdn_prefill_prepare", "gdn_prefill_scan"])
@pytest.mark.parametrize("kw,code", [
    (dict(D=64), EUNSUP),
    (dict(dt=7), EUNSUP),
    (dict(Hv=47), ESHAPE),
    (dict(Hqk=0), ESHAPE),
    (dict(T=-1), ESHAPE),
    (dict(B=-2), ESHAPE),
    (dict(q=None), ENULL),
    (dict(alpha=None), ENULL),
    (dict(o=None), ENULL),
    (dict(ws=None), EWS),
    (dict(ws_bytes=1000), EWS),
    (dict(q=addr(0, 8)), EALIGN),
    (dict(alpha=addr(3, 2)), EALIGN),
    (dict(ht=addr(7, 4)), EALIGN),
    (dict(o=addr(0, 256)), EALIAS),           # o inside q
    (dict(ht=addr(5, 1024)), EALIAS),         # ht overlaps h0 without being h0
    (dict(ws=addr(6, 4096)), EALIAS),         # workspace inside o
    (dict(ht=addr(2)), EALIAS),               # ht is v
])
def test_prefill_validation(lib, name, kw, code):
    assert prefill_call(lib, name, **kw) == code


def noalloc_call(lib, **kw):
    args = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), h0=addr(5),
                o=addr(6), ht=addr(7), B=1, T=128, Hqk=16, Hv=48, D=128, dt=BF16, stream=None)
    args.update(kw)
    return lib.gdn_prefill_chunked_noalloc(
        args["q"], args["k"], args["v"], args["alpha"], args["beta"], args["h0"], args["o"],
        args["ht"], args["B"], args["T"], args["Hqk"], args["Hv"], args["D"], args["dt"],
        args["stream"])


# Every host check of the allocation-free prefill runs before it touches the
# device, so these return on a machine without a GPU.
@pytest.mark.parametrize("kw,code", [
    (dict(D=64), EUNSUP),
    (dict(dt=7), EUNSUP),
    (dict(Hv=47), ESHAPE),
    (dict(T=-1), ESHAPE),
    (dict(q=None), ENULL),
    (dict(o=None), ENULL),
    (dict(q=addr(0, 8)), EALIGN),
    (dict(o=addr(0, 256)), EALIAS),
    (dict(ht=addr(5, 1024)), EALIAS),
    # the static scratch array holds 165 bf16 / 84 fp32 chunks of 48 value heads
    (dict(T=64 * 166), ETOOLARGE),
    (dict(B=2, T=64 * 83), ETOOLARGE),
    (dict(T=64 * 85, dt=F32), ETOOLARGE),
])
def test_noalloc_validation(lib, kw, code):
    assert noalloc_call(lib, **kw) == code


def test_noalloc_scratch_limit_matches_workspace_sizes(gdn):
    lim = 128 << 20
    assert gdn.NOALLOC_SCRATCH_BYTES == lim
    assert gdn.prefill_workspace_bytes(1, 64 * 165, 16, 48) <= lim
    assert gdn.prefill_workspace_bytes(1, 64 * 166, 16, 48) > lim
    assert gdn.prefill_workspace_bytes(1, 8192, 16, 48) <= lim      # the T = 8192 workload
    assert "GDN_ERR_TOO_LARGE" in gdn.status_str(ETOOLARGE)


def decode_call(lib, **kw):
    args = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), state=addr(5),
                o=addr(6), B=64, Hqk=16, Hv=48, D=128, dt=BF16, stream=None)
    args.update(kw)
    return lib.gdn_decode_step(args["q"], args["k"], args["v"], args["alpha"], args["beta"],
                               args["state"], args["o"], args["B"], args["Hqk"], args["Hv"],
                               args["D"], args["dt"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(D=256), EUNSUP),
    (dict(Hv=40, Hqk=16), ESHAPE),
    (dict(B=-1), ESHAPE),
    (dict(state=None), ENULL),
    (dict(beta=None), ENULL),
    (dict(v=addr(2, 4)), EALIGN),
    (dict(o=addr(5, 512)), EALIAS),           # o inside the state
    (dict(state=addr(0, 0)), EALIAS),         # state is q
])
def test_decode_validation(lib, kw, code):
    assert decode_call(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), EUNSUP),
    (dict(state=None), ENULL),
    (dict(state=addr(5, 8)), EALIGN),
    (dict(o=addr(5, 256)), EALIAS),           # o inside the bf16 state
    (dict(o=addr(5, 64 * 48 * 128 * 128 * 2 - 16)), EALIAS),   # o in the bf16 state's last bytes
])
def test_decode_bf16_state_validation(lib, kw, code):
    args = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), state=addr(5),
                o=addr(6), B=64, Hqk=16, Hv=48, D=128, dt=BF16, stream=None)
    args.update(kw)
    rc = lib.gdn_decode_step_bf16_state(args["q"], args["k"], args["v"], args["alpha"],
                                        args["beta"], args["state"], args["o"], args["B"],
                                        args["Hqk"], args["Hv"], args["D"], args["dt"],
                                        args["stream"])
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), EUNSUP),
    (dict(ht=addr(7, 4)), EALIGN),
    (dict(ht=addr(5, 1024)), EALIAS),         # ht overlaps h0 without being h0
    (dict(o=addr(5, 48 * 128 * 128 * 2 - 16)), EALIAS),   # o in h0's last bytes (bf16)
    (dict(ws=None), EWS),
])
def test_prefill_bf16_state_validation(lib, kw, code):
    assert prefill_call(lib, "gdn_prefill_chunked_bf16_state", **kw) == code


def multi_call(lib, verify=True, **kw):
    args = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), state=addr(5),
                o=addr(6), acc=addr(7), B=64, n=3, Hqk=16, Hv=48, D=128, dt=BF16, stream=None)
    args.update(kw)
    if verify:
        return lib.gdn_decode_verify(args["q"], args["k"], args["v"], args["alpha"], args["beta"],
                                     args["state"], args["o"], args["B"], args["n"], args["Hqk"],
                                     args["Hv"], args["D"], args["dt"], args["stream"])
    return lib.gdn_decode_commit(args["k"], args["v"], args["alpha"], args["beta"], args["state"],
                                 args["acc"], args["B"], args["n"], args["Hqk"], args["Hv"],
                                 args["D"], args["dt"], args["stream"])


@pytest.mark.parametrize("verify", [True, False], ids=["verify", "commit"])
@pytest.mark.parametrize("kw,code", [
    (dict(n=0), ESHAPE),
    (dict(n=9), EUNSUP),
    (dict(B=-1), ESHAPE),
    (dict(D=64), EUNSUP),
    (dict(state=None), ENULL),
    (dict(k=addr(1, 8)), EALIGN),
    (dict(beta=addr(4, 2)), EALIGN),
])
def test_verify_commit_validation(lib, verify, kw, code):
    assert multi_call(lib, verify, **kw) == code


def test_verify_commit_aliasing(lib):
    assert multi_call(lib, True, o=addr(5, 4096)) == EALIAS        # o inside the state
    assert multi_call(lib, True, o=addr(0, 64)) == EALIAS          # o inside q
    assert multi_call(lib, False, state=addr(2, 0)) == EALIAS      # state is v
    assert multi_call(lib, False, acc=None) == ENULL
    assert multi_call(lib, False, acc=addr(7, 2)) == EALIGN
    assert multi_call(lib, True, B=0) == OK and multi_call(lib, False, B=0) == OK


def test_decode_empty_batch_is_a_no_op(lib):
    assert decode_call(lib, B=0) == OK


def varlen_call(lib, **kw):
    args = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), cu=addr(9),
                N=4, T_tot=1000, h0=addr(5), o=addr(6), ht=addr(7), gate=addr(10),
                w=addr(11), eps=1e-6, Hqk=16, Hv=48, D=128, dt=BF16, ws=addr(8),
                ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return lib.gdn_prefill_varlen(args["q"], args["k"], args["v"], args["alpha"], args["beta"],
                                  args["cu"], args["N"], args["T_tot"], args["h0"], args["o"],
                                  args["ht"], args["gate"], args["w"], args["eps"], args["Hqk"],
                                  args["Hv"], args["D"], args["dt"], args["ws"],
                                  args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), EUNSUP),
    (dict(N=-1), ESHAPE),
    (dict(N=0), ESHAPE),                      # tokens but no sequences
    (dict(cu=None), ENULL),
    (dict(eps=-1.0), ESHAPE),
    (dict(eps=float("nan")), ESHAPE),
    (dict(ws_bytes=10), EWS),
    (dict(cu=addr(9, 2)), EALIGN),
    (dict(gate=addr(10, 8)), EALIGN),
    (dict(o=addr(10, 0)), EALIAS),            # o is the gate
    (dict(ws=addr(9, 0)), EALIAS),            # workspace over cu_seqlens
])
def test_varlen_validation(lib, kw, code):
    assert varlen_call(lib, **kw) == code


def test_varlen_empty_is_a_no_op(lib):
    assert varlen_call(lib, N=0, T_tot=0) == OK


def test_binding_rejects_bad_tensors(gdn):
    import torch
    q = torch.zeros(1, 64, 16, 128)
    with pytest.raises(ValueError):
        gdn.prefill_chunked(q, q, torch.zeros(1, 64, 48, 64), torch.zeros(1, 64, 48),
                            torch.zeros(1, 64, 48))
    with pytest.raises(TypeError):
        gdn.prefill_chunked(q.half(), q.half(), torch.zeros(1, 64, 48, 128).half(),
                            torch.zeros(1, 64, 48), torch.zeros(1, 64, 48))
    with pytest.raises(ValueError):
        gdn.decode_step(torch.zeros(2, 16, 128), torch.zeros(2, 16, 128), torch.zeros(2, 48, 128),
                        torch.zeros(2, 48), torch.zeros(2, 48), torch.zeros(2, 48, 128, 64))


def bwd_call(lib, **kw):
    args = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), h0=addr(5),
                do=addr(6), dht=addr(7), dq=addr(8), dk=addr(9), dv=addr(10), da=addr(11),
                db=addr(12), dh0=addr(13), B=1, T=128, Hqk=16, Hv=48, D=128, dt=BF16,
                ws=addr(14), ws_bytes=1 << 40, stream=None)
    args.update(kw)
    a = args
    return lib.gdn_prefill_chunked_bwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["h0"],
                                       a["do"], a["dht"], a["dq"], a["dk"], a["dv"], a["da"],
                                       a["db"], a["dh0"], a["B"], a["T"], a["Hqk"], a["Hv"],
                                       a["D"], a["dt"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), EUNSUP),
    (dict(dt=7), EUNSUP),
    (dict(Hv=47), ESHAPE),
    (dict(T=-1), ESHAPE),
    (dict(do=None), ENULL),
    (dict(dq=None), ENULL),
    (dict(db=None), ENULL),
    (dict(ws=None), EWS),
    (dict(ws_bytes=1000), EWS),
    (dict(do=addr(6, 8)), EALIGN),
    (dict(dh0=addr(13, 4)), EALIGN),
    (dict(da=addr(11, 2)), EALIGN),
    (dict(dq=addr(0, 512)), EALIAS),          # dq inside q
    (dict(dv=addr(8, 256)), EALIAS),          # dv inside dq
    (dict(dh0=addr(7)), EALIAS),              # dh0 is dht
    (dict(ws=addr(10, 4096)), EALIAS),        # workspace inside dv
])
def test_backward_validation(lib, kw, code):
    assert bwd_call(lib, **kw) == code


def test_backward_workspace_and_empty_batch(gdn, lib):
    # per chunk: the forward workspace, N (48 x 64 x 64) and two 48 x 128 x 128
    # state stacks, bf16
    w1 = gdn.prefill_bwd_workspace_bytes(1, 64, 16, 48)
    w2 = gdn.prefill_bwd_workspace_bytes(1, 128, 16, 48)
    fwd = gdn.prefill_workspace_bytes(1, 128, 16, 48) - gdn.prefill_workspace_bytes(1, 64, 16, 48)
    assert w2 - w1 == fwd + 48 * 4096 * 2 + 2 * 48 * 128 * 128 * 2
    assert gdn.prefill_bwd_workspace_bytes(1, 0, 16, 48) == 0
    assert gdn.prefill_bwd_workspace_bytes(1, 64, 16, 48, D=64) == 0
    assert bwd_call(lib, B=0) == OK


def attn_prefill_call(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), gate=addr(3), qw=addr(4), kw=addr(5), eps=1e-6,
             o=addr(6), kc=addr(7), vc=addr(8), cache_len=256, B=1, T=128, Hq=24, Hkv=4, D=256,
             rope=64, theta=1e7, dt=BF16, ws=addr(9), ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.gdn_attn_prefill(a["q"], a["k"], a["v"], a["gate"], a["qw"], a["kw"], a["eps"],
                                a["o"], a["kc"], a["vc"], a["cache_len"], a["B"], a["T"], a["Hq"],
                                a["Hkv"], a["D"], a["rope"], a["theta"], a["dt"], a["ws"],
                                a["ws_bytes"], a["stream"])


def attn_decode_call(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), gate=addr(3), qw=addr(4), kw=addr(5), eps=1e-6,
             o=addr(6), kc=addr(7), vc=addr(8), pos=addr(10), cache_len=256, B=4, Hq=24, Hkv=4,
             D=256, rope=64, theta=1e7, dt=BF16, ws=addr(9), ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.gdn_attn_decode(a["q"], a["k"], a["v"], a["gate"], a["qw"], a["kw"], a["eps"],
                               a["o"], a["kc"], a["vc"], a["pos"], a["cache_len"], a["B"], a["Hq"],
                               a["Hkv"], a["D"], a["rope"], a["theta"], a["dt"], a["ws"],
                               a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(D=128), EUNSUP),
    (dict(Hq=25), ESHAPE),
    (dict(Hq=48), EUNSUP),                    # 12 query heads per key/value head
    (dict(rope=60), EUNSUP),
    (dict(rope=264), EUNSUP),
    (dict(theta=0.0), ESHAPE),
    (dict(eps=-1.0), ESHAPE),
    (dict(T=-1), ESHAPE),
    (dict(dt=5), EUNSUP),
    (dict(q=None), ENULL),
    (dict(gate=None), ENULL),
    (dict(vc=None), ENULL),                   # caches come in pairs
    (dict(cache_len=100), ESHAPE),            # cache shorter than the prompt
    (dict(ws=None), EWS),
    (dict(ws_bytes=4096), EWS),
    (dict(q=addr(0, 8)), EALIGN),
    (dict(qw=addr(4, 2)), EALIGN),
    (dict(o=addr(0, 512)), EALIAS),           # o inside q
    (dict(kc=addr(6)), EALIAS),               # key cache is o
    (dict(ws=addr(8, 1024)), EALIAS),         # workspace inside the value cache
])
def test_attn_prefill_validation(lib, kw, code):
    assert attn_prefill_call(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(D=128), EUNSUP),
    (dict(cache_len=0), ESHAPE),
    (dict(pos=None), ENULL),
    (dict(kc=None), ENULL),
    (dict(pos=addr(10, 2)), EALIGN),
    (dict(o=addr(3, 64)), EALIAS),            # o inside the gate
    (dict(ws=None), EWS),
])
def test_attn_decode_validation(lib, kw, code):
    assert attn_decode_call(lib, **kw) == code


def test_attn_empty_calls_and_workspace(gdn, lib):
    assert attn_prefill_call(lib, T=0) == OK and attn_prefill_call(lib, B=0) == OK
    assert attn_decode_call(lib, B=0) == OK
    # prefill: rotated queries and keys in the element type
    assert gdn.attn_prefill_workspace_bytes(1, 64) == 64 * 24 * 256 * 2 + 64 * 4 * 256 * 2
    # decode: rotated queries, then per 512-key split a max, a sum and 256 fp32
    def r256(x):
        return (x + 255) // 256 * 256

    # splits: about 512 workgroups over the B * 4 streams, multiples of 32 keys
    for B, L, ns in ((2, 512, 16), (2, 8192, 64), (64, 8192, 2), (64, 100, 2), (1, 40, 2)):
        want = r256(B * 24 * 256 * 2) + 2 * r256(B * 24 * ns * 4) + r256(B * 24 * ns * 256 * 4)
        assert gdn.attn_decode_workspace_bytes(B, L) == want, (B, L)
    assert gdn.attn_decode_workspace_bytes(2, 0) == 0


def varlen_bwd_call(lib, **kw):
    a = dict(q=addr(0), k=addr(1), v=addr(2), alpha=addr(3), beta=addr(4), cu=addr(15), N=3,
             T=300, h0=addr(5), do=addr(6), dht=addr(7), dq=addr(8), dk=addr(9), dv=addr(10),
             da=addr(11), db=addr(12), dh0=addr(13), Hqk=16, Hv=48, D=128, dt=BF16, ws=addr(14),
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.gdn_prefill_varlen_bwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["cu"],
                                      a["N"], a["T"], a["h0"], a["do"], a["dht"], a["dq"],
                                      a["dk"], a["dv"], a["da"], a["db"], a["dh0"], a["Hqk"],
                                      a["Hv"], a["D"], a["dt"], a["ws"], a["ws_bytes"],
                                      a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), EUNSUP),
    (dict(N=-1), ESHAPE),
    (dict(N=0), ESHAPE),                      # tokens without sequences
    (dict(cu=None), ENULL),
    (dict(do=None), ENULL),
    (dict(ws=None), EWS),
    (dict(cu=addr(15, 2)), EALIGN),
    (dict(dk=addr(1, 256)), EALIAS),          # dk inside k
    (dict(ws=addr(15)), EALIAS),              # workspace is cu_seqlens
])
def test_varlen_backward_validation(lib, kw, code):
    assert varlen_bwd_call(lib, **kw) == code


def test_varlen_backward_workspace(gdn, lib):
    assert varlen_bwd_call(lib, N=0, T=0) == OK
    # the fixed-length layout for ceil(T/64) + N chunks, plus the chunk table
    w = gdn.varlen_bwd_workspace_bytes(3, 300, 16, 48)
    assert w > gdn.prefill_bwd_workspace_bytes(1, 64 * 8, 16, 48)
    assert gdn.varlen_bwd_workspace_bytes(3, 300, 16, 48, D=64) == 0
