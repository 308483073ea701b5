"""Benchmark of the Gated DeltaNet recurrence on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--decode-steps S] [--no-other-workloads] [--copy-calibration]

One step = one chunked prefill call of the T = 8192 workload (batch 1, 16
query/key heads, 48 value heads, head dim 128, bf16 q/k/v, fp32 gates, zero
initial state, final state emitted): the prepare kernel followed by the scan
kernel, on inputs already resident in HBM.  The decode workload (64 sequences
x 1 token, fp32 state 64 x 48 x 128 x 128 updated in place) is timed in the
same run and reported under "decode"; so are the other prefill workloads
(fp32 T = 256; T = 262,144 with a carried state; the packed batch of 8
sequences of 1,024 .. 32,768 tokens, plain and with the gated RMSNorm
epilogue), the backward of the T = 8192 call and the gated attention layer.
Prints one JSON line.

Rates:
* prefill: tokens/s = T / step time; TFLOP/s from the method's algorithmic
  FLOP count per call (below), against the dense bf16 MFMA peak;
* decode: state GB/s = 2 x 64 x 48 x 128 x 128 x 4 bytes / step time,
  against the HBM peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

import synth

D, C, HQK, HV = 128, 64, 16, 48
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E


def prefill_flops(T, B=1):
    """Algorithmic FLOPs of one chunked prefill call: per chunk and value head
    6Cd^2 + 6C^2d + C^3/3, plus 4C^2d per chunk and query/key head (the two
    Gram matrices, shared by the value heads of the group)."""
    nc = B * ((T + C - 1) // C)
    return nc * (HV * (6 * C * D * D + 6 * C * C * D + C ** 3 / 3) + HQK * 4 * C * C * D)


def scan_flops(T, B=1):
    """Algorithmic FLOPs of the scan kernel per launch: per chunk and value
    head, K S^T, Q S^T and the state update (2Cd^2 each) plus Tt X and M Dl
    (2C^2d each)."""
    nc = B * ((T + C - 1) // C)
    return nc * HV * (6 * C * D * D + 4 * C * C * D)


def backward_flops(T, B=1):
    """Algorithmic FLOPs of one backward call (gdn_prefill_chunked_bwd), per
    chunk and value head: the state-checkpoint pass 4Cd^2 + 2C^2d, the reverse
    state-gradient chain 6Cd^2 + 4C^2d, the per-chunk gradients 10Cd^2 +
    16C^2d, the in-chunk solve C^3/3; per chunk and query/key head the Gram
    matrices of prepare and of the gradient kernel, 8C^2d."""
    nc = B * ((T + C - 1) // C)
    return nc * (HV * (20 * C * D * D + 22 * C * C * D + C ** 3 / 3) + HQK * 8 * C * C * D)


def grad_kernel_flops(T, B=1):
    """Algorithmic FLOPs of the per-chunk gradient kernel per launch."""
    nc = B * ((T + C - 1) // C)
    return nc * HV * (10 * C * D * D + 16 * C * C * D)


def decode_state_bytes(B):
    return 2 * B * HV * D * D * 4


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_bytes_bench_workloads.md")


def sources_hash(names):
    """sha256 over the concatenated bytes of the listed csrc files (a kernel's
    source and every header it includes), or None if one is missing."""
    h = hashlib.sha256()
    try:
        for n in names.split(","):
            h.update(open(os.path.join(ROOT, "hybrid_linear_attention_amd", "csrc", n), "rb").read())
    except OSError:
        return None
    return h.hexdigest()


def counted_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (calibrated against a plain copy), or None
    when there is no such line or the kernel's sources have changed since the
    counters were taken."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) == 5 and f[0] == "traffic" and f[1] == kernel:
            return int(f[4]) if sources_hash(f[2]) == f[3] else None
    return None


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_ops_bench_workloads.md")


def counted_mfma_gflop():
    """Matrix-unit FLOPs one prefill call executes, from the committed
    rocprofv3 SQ_INSTS_VALU_MFMA_* summary (per prepare + scan call), or None
    when the summary is absent or the prefill source changed since."""
    try:
        lines = open(MFMA_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) == 5 and f[0] == "mfma_gflop" and f[1] == "prefill":
            return float(f[4]) if sources_hash(f[2]) == f[3] else None
    return None


def scan_bytes(T, B=1):
    """Algorithmic bytes of one scan launch (bf16): it reads q, v, the
    workspace (Tt and M: 64 x 64 bf16 per chunk and value head; K^T: 128 x 64
    bf16 per chunk and query/key head; two fp32 gate vectors of 64 per chunk and
    value head) and writes o and the fp32 final state."""
    nc = B * ((T + C - 1) // C)
    tok = B * T
    rd = tok * HQK * D * 2 + tok * HV * D * 2 + nc * (HV * 2 * C * C * 2 + HQK * D * C * 2 + HV * 2 * C * 4)
    wr = tok * HV * D * 2 + B * HV * D * D * 4
    return rd + wr


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_prefill(gdn, inp, steps, warmup):
    dev = inp["q"].device
    T = inp["q"].shape[1]
    o = torch.empty((1, T, HV, D), dtype=inp["q"].dtype, device=dev)
    ht = torch.empty((1, HV, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(1, T, HQK, HV, D, inp["q"].dtype),
                     dtype=torch.uint8, device=dev)
    args = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp.get("h0"), o, ht, ws)
    for _ in range(warmup):
        gdn.prefill_prepare(*args)
        gdn.prefill_scan(*args)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        gdn.prefill_prepare(*args)
        ev[i][1].record(stream)
        gdn.prefill_scan(*args)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    scan = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    step = ev[0][0].elapsed_time(ev[-1][2]) / steps
    per_call = sorted(e[0].elapsed_time(e[2]) for e in ev)

    def pct(p):
        return per_call[min(len(per_call) - 1, int(round(p * (len(per_call) - 1))))]

    return dict(step_ms=step, prepare_ms=prep, scan_ms=scan, wall_s=wall,
                median_ms=pct(0.5), p10_ms=pct(0.1), p90_ms=pct(0.9))


def timed_decode(gdn, B, steps, warmup, dtype=torch.bfloat16, state_dtype=torch.float32):
    dev = "cuda:0"
    state = synth.decode_state(B, 1002, 0.02).to(state_dtype).to(dev)
    sets = [{k: v.to(dev) for k, v in synth.decode_step_inputs(B, s, dtype, seed=1002).items()}
            for s in range(4)]
    o = torch.empty((B, HV, D), dtype=dtype, device=dev)

    def step(i):
        d = sets[i % len(sets)]
        gdn.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], state, o=o)

    for i in range(warmup):
        step(i)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = decode_state_bytes(B) * state.element_size() // 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(step_ms=ms, gbs=gbs, state_bytes=nbytes)


def timed_speculative(gdn, B, n, rounds, warmup):
    """Verify of n drafted tokens then commit of all of them, per round: the
    state is read by verify and read + written by commit."""
    dev = "cuda:0"
    state = synth.decode_state(B, 1002, 0.02).to(dev)
    d = {k: v.to(dev) for k, v in synth.prefill_inputs(B, n, torch.bfloat16, seed=77).items()
         if v is not None}
    acc = torch.full((B,), n, dtype=torch.int32, device=dev)
    o = torch.empty((B, n, HV, D), dtype=torch.bfloat16, device=dev)

    def rnd():
        gdn.decode_verify(d["q"], d["k"], d["v"], d["alpha"], d["beta"], state, o=o)
        gdn.decode_commit(d["k"], d["v"], d["alpha"], d["beta"], state, acc)

    for _ in range(warmup):
        rnd()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(rounds):
        rnd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / rounds
    nbytes = 3 * decode_state_bytes(B) // 2
    return dict(ms=ms, gbs=nbytes / (ms * 1e-3) / 1e9, tokens_per_s=B * n / (ms * 1e-3))


def timed_backward(gdn, T, steps, warmup):
    """One backward call of the T-token bf16 training shape (zero initial
    state, no final-state gradient), inputs and workspace resident."""
    d = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v)
         for k, v in synth.backward_inputs(1, T, torch.bfloat16, seed=1011).items()}
    ws = torch.empty(gdn.prefill_bwd_workspace_bytes(1, T, HQK, HV, D, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["do"], None, None)
    g = gdn.prefill_backward(*args, workspace=ws)
    for _ in range(warmup):
        gdn.prefill_backward(*args, grads=g, workspace=ws)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        gdn.prefill_backward(*args, grads=g, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return dict(ms=ms, tokens_per_s=T / (ms * 1e-3),
                tflops=backward_flops(T) / (ms * 1e-3) / 1e12)


ATT_HQ, ATT_HKV, ATT_D = 24, 4, 256


def attention_prefill_flops(T, B=1):
    """Algorithmic FLOPs of a causal gated-attention prefill: Q K^T and P V over
    the T (T + 1) / 2 query-key pairs of every query head, 2 FLOPs per
    multiply-add each."""
    return B * ATT_HQ * 4 * ATT_D * T * (T + 1) / 2


def attention_decode_bytes(B, n):
    """Algorithmic bytes of one decode step over n cached keys per sequence:
    the bf16 keys and values read once (the query, gate, output and the new
    key/value row are under 0.1 % of it)."""
    return B * n * ATT_HKV * ATT_D * 2 * 2


def timed_attention(gdn, T, Bd, Ld, steps):
    """Gated attention layer: a T-token prefill (batch 1) and a decode step of
    Bd sequences with Ld - 1 cached keys each (bf16)."""
    d = {k: v.to("cuda") for k, v in synth.attention_inputs(1, T, torch.bfloat16, seed=1201).items()}
    ws = torch.empty(gdn.attn_prefill_workspace_bytes(1, T), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(d["q"])

    def pre():
        gdn.attn_prefill(d["q"], d["k"], d["v"], d["gate"], d["q_norm_w"], d["k_norm_w"], o=o,
                         workspace=ws)

    g = torch.Generator().manual_seed(1202)
    kc = torch.randn((Bd, Ld, ATT_HKV, ATT_D), generator=g).to(torch.bfloat16).to("cuda")
    vc = torch.randn((Bd, Ld, ATT_HKV, ATT_D), generator=g).to(torch.bfloat16).to("cuda")
    s = {k: v.to("cuda") for k, v in synth.attention_decode_inputs(Bd, 0, torch.bfloat16,
                                                                    seed=1203).items()}
    pos = torch.full((Bd,), Ld - 1, dtype=torch.int32, device="cuda")
    wsd = torch.empty(gdn.attn_decode_workspace_bytes(Bd, Ld), dtype=torch.uint8, device="cuda")
    od = torch.empty_like(s["q"])

    def dec():
        gdn.attn_decode(s["q"], s["k"], s["v"], s["gate"], kc, vc, pos, d["q_norm_w"],
                        d["k_norm_w"], o=od, workspace=wsd)

    res = {}
    stream = torch.cuda.current_stream()
    for name, fn in (("prefill", pre), ("decode", dec)):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    return res


def cpu_baseline(inp, T_sample, min_seconds=10.0, max_calls=64):
    """The float64 oracle, untuned, on the same workload: the first T_sample
    tokens of every value head, called repeatedly until about min_seconds of
    CPU work have run (each call is independent; the rate is tokens over the
    summed wall time)."""
    import oracle
    oracle.build(force=False)
    sl = {k: inp[k][:, :T_sample].cpu() for k in ("q", "k", "v", "alpha", "beta")}
    threads = oracle.num_threads()               # team size of the oracle's parallel region
    calls, dt = 0, 0.0
    while calls < max_calls and dt < min_seconds:
        t0 = time.perf_counter()
        oracle.prefill(sl["q"], sl["k"], sl["v"], sl["alpha"], sl["beta"], None)
        dt += time.perf_counter() - t0
        calls += 1
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rate = calls * T_sample / dt
    single = cpu_single_thread()
    return dict(value=rate, unit="tokens/s", cores=threads, kind="oracle",
                sample="%d calls on the first %d of 8192 tokens, all 48 value heads, batch 1, "
                       "float64 sequential recurrence, OpenMP over heads (%.1f s)"
                       % (calls, T_sample, dt),
                cpu_model=model, single_thread=single,
                # per-token work does not depend on T, so the two rates compare
                # directly: this is the speed-up the host actually gave the threads
                parallel_speedup=(rate / single["value"]) if single.get("value") else None)


def cpu_single_thread(T_sample=256):
    """The same oracle on one core: a child process pinned to one CPU
    (sched_setaffinity before anything loads OpenMP) that calls the oracle one
    value head at a time (oracle.subset_heads), so that each call holds a
    single chain and one thread does all the work whatever team size the
    OpenMP runtime uses; the first T_sample tokens of all 48 heads, repeated
    for about five seconds.  It reports the team size the oracle's parallel
    region ran with (a team larger than one shares the one CPU and has one
    chain to run)."""
    import subprocess
    code = ("import os\n"
            "cpu = sorted(os.sched_getaffinity(0))[0]\n"
            "os.sched_setaffinity(0, {cpu})\n"
            "import time, synth, oracle\n"
            "oracle.build(force=False)\n"
            "oracle.set_num_threads(1)\n"
            "d = synth.config_inputs(1)\n"
            "sl = {k: d[k][:, :%d] for k in ('q', 'k', 'v', 'alpha', 'beta')}\n"
            "subs = [oracle.subset_heads(sl['q'], sl['k'], sl['v'], sl['alpha'], sl['beta'], None,\n"
            "                            [h], 16, 48) for h in range(48)]\n"
            "n, t = 0, 0.0\n"
            "while t < 5.0 and n < 64:\n"
            "    t0 = time.perf_counter()\n"
            "    for sub in subs:\n"
            "        oracle.prefill(*sub)\n"
            "    t += time.perf_counter() - t0\n"
            "    n += 1\n"
            "print(n * %d / t, oracle.num_threads(), len(os.sched_getaffinity(0)))\n"
            % (T_sample, T_sample))
    env = dict(os.environ, OMP_NUM_THREADS="1", OMP_WAIT_POLICY="PASSIVE", GOMP_SPINCOUNT="0",
               CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    try:
        out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                             text=True, timeout=120)
        rate, nthr, ncpu = out.stdout.strip().splitlines()[-1].split()
        return dict(value=float(rate), unit="tokens/s", cores=int(ncpu), team_size=int(nthr),
                    sample="first %d of 8192 tokens, all 48 value heads one head per call, "
                           "float64, pinned to one CPU" % T_sample)
    except Exception as e:  # reported, never fatal: it is a side figure
        return dict(value=None, error=str(e)[:200])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the fp32 T=256, T=262,144 and packed varlen prefill figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    from hybrid_linear_attention_amd import gdn

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written")

    cfg = synth.CONFIGS[1]
    T = cfg["T"]
    inp_cpu = synth.config_inputs(1)
    inp = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp_cpu.items()}
    log("prefill T=%d: warmup %d, steps %d" % (T, args.warmup, args.steps))
    pre = timed_prefill(gdn, inp, args.steps, args.warmup)
    log("prefill step %.3f ms (prepare %.3f, scan %.3f)" %
        (pre["step_ms"], pre["prepare_ms"], pre["scan_ms"]))
    tok_s = T / (pre["step_ms"] * 1e-3)
    tflops = prefill_flops(T) / (pre["step_ms"] * 1e-3) / 1e12

    dominant = "scan" if pre["scan_ms"] >= pre["prepare_ms"] else "prepare"
    scan_tflops = scan_flops(T) / (pre["scan_ms"] * 1e-3) / 1e12

    log("decode B=64: %d steps" % args.decode_steps)
    dec = timed_decode(gdn, 64, args.decode_steps, 16)
    log("decode step %.4f ms, %.1f GB/s" % (dec["step_ms"], dec["gbs"]))
    # 64 x 48 x 128 x 128 fp32 (192 MiB) fits in the 256 MB last-level cache;
    # 256 sequences (768 MiB) do not, which shows the rate that DRAM sustains.
    log("decode B=256 (state larger than the last-level cache): 64 steps")
    dec256 = timed_decode(gdn, 256, 64, 8)
    log("decode B=256 step %.4f ms, %.1f GB/s" % (dec256["step_ms"], dec256["gbs"]))
    log("decode B=64 with the state stored in bf16: %d steps" % args.decode_steps)
    decb = timed_decode(gdn, 64, args.decode_steps, 16, state_dtype=torch.bfloat16)
    log("decode bf16-state step %.4f ms, %.1f GB/s" % (decb["step_ms"], decb["gbs"]))
    spec = timed_speculative(gdn, 64, 3, 64, 8)
    log("speculative verify + commit of 3 tokens x 64 sequences: %.4f ms, %.1f GB/s"
        % (spec["ms"], spec["gbs"]))

    log("backward T=%d (training shape): 20 calls" % T)
    bwd = timed_backward(gdn, T, 20, 3)
    log("backward %.3f ms, %.2f M tokens/s, %.1f TFLOP/s" %
        (bwd["ms"], bwd["tokens_per_s"] / 1e6, bwd["tflops"]))

    log("gated attention layer: prefill T=%d, decode 64 x 8192 keys" % T)
    att = timed_attention(gdn, T, 64, 8192, 20)
    att_tf = attention_prefill_flops(T) / (att["prefill"] * 1e-3) / 1e12
    att_gbs = attention_decode_bytes(64, 8192) / (att["decode"] * 1e-3) / 1e9
    log("attention prefill %.3f ms (%.1f TFLOP/s), decode %.4f ms (%.1f GB/s)"
        % (att["prefill"], att_tf, att["decode"], att_gbs))

    out = {
        "metric": "GDN prefill tokens/s @T=8192 (% MFMA peak) + decode state GB/s (% HBM peak)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chunked prefill, batch 1, T=8192, 16 QK / 48 V heads, head "
                               "dim 128, chunk 64, bf16 q/k/v, fp32 alpha/beta/state, "
                               "zero initial state, final state emitted",
                   "global_batch": 1, "seq_len": T, "parallelism": "single GPU"},
        "prefill": {"tflops_algorithmic": tflops, "frac_bf16_mfma_peak": tflops / PEAK_BF16_TFLOPS,
                    "prepare_ms": pre["prepare_ms"], "scan_ms": pre["scan_ms"],
                    "per_call_ms": {"median": pre["median_ms"], "p10": pre["p10_ms"],
                                    "p90": pre["p90_ms"]},
                    "gflop_per_call": prefill_flops(T) / 1e9,
                    "mfma_gflop_counted": counted_mfma_gflop()},
        "roofline": {"bound": "mfma", "kernel": dominant,
                     "achieved": scan_tflops if dominant == "scan" else None,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": (scan_tflops / PEAK_BF16_TFLOPS) if dominant == "scan" else None,
                     "traffic": counted_traffic("scan_split_kernel<false>") if dominant == "scan" else None,
                     "algorithmic_bytes": scan_bytes(T),
                     "hbm_gbs": scan_bytes(T) / (pre["scan_ms"] * 1e-3) / 1e9},
        "decode": {"metric": "decode state GB/s", "value": dec["gbs"], "unit": "GB/s",
                   "ms_per_step": dec["step_ms"], "steps": args.decode_steps,
                   "workload": "64 sequences x 1 token, fp32 state [64,48,128,128] in place, "
                               "bf16 q/k/v",
                   "roofline": {"bound": "hbm", "achieved": dec["gbs"], "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": dec["gbs"] / PEAK_HBM_GBS,
                                "traffic": counted_traffic("decode_step_kernel@B64")},
                   "dram_diagnostic_B256": {"ms_per_step": dec256["step_ms"], "gbs": dec256["gbs"],
                                            "frac": dec256["gbs"] / PEAK_HBM_GBS},
                   "bf16_state": {"ms_per_step": decb["step_ms"], "gbs": decb["gbs"],
                                  "frac": decb["gbs"] / PEAK_HBM_GBS,
                                  "state_bytes_per_step": decb["state_bytes"],
                                  "sequences_per_s": 64 / (decb["step_ms"] * 1e-3)},
                   "speculative_n3": {"ms_per_round": spec["ms"], "state_gbs": spec["gbs"],
                                      "frac": spec["gbs"] / PEAK_HBM_GBS,
                                      "tokens_per_s_all_accepted": spec["tokens_per_s"],
                                      "workload": "64 sequences, verify of 3 drafted tokens then "
                                                  "commit of all 3, fp32 state"}},
    }
    out["backward"] = {
        "workload": "gradients of the T=8192 prefill (dq, dk, dv, dalpha, dbeta, dh0), bf16, "
                    "zero initial state, upstream gradient of o only",
        "ms_per_call": bwd["ms"], "tokens_per_s": bwd["tokens_per_s"],
        "tflops_algorithmic": bwd["tflops"], "frac_bf16_mfma_peak": bwd["tflops"] / PEAK_BF16_TFLOPS,
        "gflop_per_call": backward_flops(T) / 1e9,
        "grad_kernel_gflop_per_launch": grad_kernel_flops(T) / 1e9}
    out["attention"] = {
        "workload": "gated attention layer (24 query / 4 key-value heads, head dim 256, "
                    "QK-Norm, RoPE on 64 channels with theta 1e7, causal, sigmoid output gate), "
                    "bf16; prefill batch 1 T=8192; decode 64 sequences x 8192 cached keys",
        "prefill": {"ms": att["prefill"], "tokens_per_s": T / (att["prefill"] * 1e-3),
                    "tflops_algorithmic": att_tf, "frac_bf16_mfma_peak": att_tf / PEAK_BF16_TFLOPS,
                    "gflop_per_call": attention_prefill_flops(T) / 1e9},
        "decode": {"ms_per_step": att["decode"], "gbs": att_gbs, "frac": att_gbs / PEAK_HBM_GBS,
                   "cache_bytes_per_step": attention_decode_bytes(64, 8192),
                   "roofline": {"bound": "hbm", "achieved": att_gbs, "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": att_gbs / PEAK_HBM_GBS,
                                "traffic": counted_traffic("attn_decode_kernel")}}}
    if not args.no_other_workloads:
        log("fp32 prefill, T=256")
        inp0 = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v)
                for k, v in synth.config_inputs(0).items()}
        r0 = timed_prefill(gdn, inp0, 100, 10)
        out["config0_fp32_T256"] = {"median_ms": r0["median_ms"], "p10_ms": r0["p10_ms"],
                                    "p90_ms": r0["p90_ms"],
                                    "tokens_per_s": 256 / (r0["median_ms"] * 1e-3)}
        del inp0
        log("bf16 prefill, T=262144, carried state")
        inp3 = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v)
                for k, v in synth.config_inputs(3).items()}
        r3 = timed_prefill(gdn, inp3, 10, 3)
        out["long_context"] = {"T": 262144, "ms": r3["step_ms"],
                               "tokens_per_s": 262144 / (r3["step_ms"] * 1e-3),
                               "tflops_algorithmic": prefill_flops(262144) / (r3["step_ms"] * 1e-3) / 1e12}
        del inp3
        log("packed varlen batch, plain and with the gated RMSNorm epilogue")
        inp4 = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v)
                for k, v in synth.config_inputs(4).items()}
        T4 = int(inp4["cu_seqlens"][-1].item())
        res = {}
        for gated in (False, True):
            vargs = (inp4["q"], inp4["k"], inp4["v"], inp4["alpha"], inp4["beta"],
                    inp4["cu_seqlens"], inp4["h0"])
            kw = dict(gate=inp4["gate"]) if gated else {}
            for _ in range(3):
                gdn.prefill_varlen(*vargs, **kw)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                gdn.prefill_varlen(*vargs, **kw)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            res["gated" if gated else "plain"] = {"ms": ms, "tokens_per_s": T4 / (ms * 1e-3)}
            log("varlen %s: %.3f ms, %.1f M tokens/s" % ("gated" if gated else "plain", ms,
                                                         T4 / ms / 1e3))
        res["plain"]["traffic"] = counted_traffic("scan_head_kernel<false>")
        res["gated"]["traffic"] = counted_traffic("scan_head_kernel<true>")
        out["varlen_8_sequences"] = dict(tokens=T4, lengths=[int(x) for x in inp4["lengths"]],
                                         scan="head-wide (one workgroup per head and sequence)",
                                         **res)
        del inp4
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on %d tokens" % args.cpu_tokens)
        out["cpu_baseline"] = cpu_baseline(inp_cpu, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
