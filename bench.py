#!/usr/bin/env python3
"""One-GPU benchmark of the attention hot path (forward + recompute backward).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-rows-f] [--no-oracle]

A step is one forward (fa_fwd) and one backward (fa_bwd: D = rowsum(dO*O),
dK/dV, dQ) over the long-context workload: B=1, H=16, N=16384, d=128, bf16,
causal, inputs iid N(0,1) * 0.5, dO iid N(0,1), all resident in HBM before
timing starts.  FLOPs follow the usual convention: forward 4*B*H*Nq*Nk*d,
halved when causal; backward 2.5x the forward.  Prints ONE JSON line on
stdout; human-readable detail goes to stderr.

Timing: W untimed warm-up steps, then exactly K steps between
torch.cuda.synchronize() calls, with HIP events recorded on the launch stream
around every forward and backward call.  Afterwards each backward stage is
timed alone (K launches each, via fa_bwd_stages) so every kernel has its own
event-measured average duration; the dominant one is reported as `roofline`
(and the forward kernel, the long-context target, as `roofline_fwd`).

rows_f: the same step for the built extensions on the same inputs: 16 query
heads on 2 K/V heads (causal), a causal sliding window of 256 keys (the skill
guide's window example), and causal dropout with p = 0.1 (the skill guide's
dropout_p); the plain step on 2 of the 16 heads (one GPU's share under 8-way
head sharding); plus the fp8 forward alone on the inputs cast to float8_e4m3fn
(priced against the fp8 MFMA peak, 5.0 PFLOP/s).  FLOPs count admitted
(query, key) pairs.

cpu_baseline: the fp64 numpy oracle (test infrastructure) on four heads of the
same workload, forward + backward, timed on the host cores.

configs: the per-configuration report.  The four smaller workloads
(forward; forward and backward for the training-step one), timed per launch
from a replayed HIP graph and from a Python loop, at the clock sampled while
each runs back to back, with parity against the oracle on the same seeded
inputs, the oracle's host time, and MFMA busy / HBM GB/s from the committed
counter summary; the 16K workload's entry (parity on 256 sampled rows per
head and on the cpu_baseline heads); and a chip-filling non-causal row (the
16K inputs without the mask).

power_context: under load the chip runs at its power cap and lowers its
clock; the forward is run back to back for a few seconds while amd-smi reads
the GFX clock and socket power, and so is a bf16 GEMM of 8192^3 (torch.matmul
on random operands) as the dense-MFMA rate a tuned library reaches under
the same cap.
"""
import argparse
import hashlib
import re
import json
import math
import os
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp8": 5000.0}  # MI355X dense MFMA, published
PEAK_HBM_GBS = 8000.0
WORKLOAD = "fwd_causal_b1h16_n16384_d128_bf16_bhsd"
METRIC = "attention fwd/bwd TFLOP/s + % of MFMA peak (fp16/bf16, causal & not)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_causal_b1h16_n16384_d128_bf16.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the kernel sources' code with comments and whitespace
    removed: a change of a comment leaves the counters valid, a change of
    code does not."""
    h = hashlib.sha256()
    for f in ("fa_device.h", "fa_kernels.h", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip"):
        with open(os.path.join(ROOT, "exact_io_aware_02_amd", "csrc", f), encoding="utf-8") as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def smi_sample():
    """(mean GFX clock in MHz over the XCDs, socket power in W) read with
    amd-smi in a child process, or None where it is unavailable."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--power", "--clock", "--json"],
                           capture_output=True, text=True, timeout=30)
        txt = r.stdout
        d, _ = json.JSONDecoder().raw_decode(txt[txt.index("["):])
        g = d[0]
        clks = [v["clk"]["value"] for kk, v in g["clock"].items()
                if kk.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        return float(sum(clks)) / len(clks), float(g["power"]["socket_power"]["value"])
    except Exception:
        return None


def sustained(torch, fn, seconds, stream):
    """Run fn back to back for about `seconds` while a second thread samples
    the clock and power twice; returns (ms per call, MHz, W)."""
    samples = []

    def sampler():
        time.sleep(min(1.5, seconds / 3))
        for _ in range(2):
            x = smi_sample()
            if x is not None:
                samples.append(x)
            time.sleep(0.3)

    th = threading.Thread(target=sampler)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    th.start()
    t0 = time.perf_counter()
    n = 0
    e0.record(stream)
    while n == 0 or th.is_alive() or time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    e1.record(stream)
    torch.cuda.synchronize()
    th.join()
    ms = e0.elapsed_time(e1) / n
    if not samples:
        return ms, None, None
    return ms, sum(x[0] for x in samples) / len(samples), sum(x[1] for x in samples) / len(samples)


def power_context(torch, fa, q, k, v, o, lse, s, causal, stream, fwd_flop, peak):
    """The chip's power cap sets its clock under load: the forward back to
    back with amd-smi's clock and power readings, beside a large bf16 GEMM
    (torch.matmul, hipBLASLt) on random N(0,1) operands as the dense-MFMA
    rate a tuned library reaches under the same cap, and the same GEMM on
    e4m3 operands (torch._scaled_mm) for the fp8 forward's row."""
    out = {}
    ms, mhz, w = sustained(torch, lambda: fa.fa_fwd(q, k, v, o, lse, s, causal, stream), 4.0, stream)
    tf = fwd_flop / ms / 1e9
    out["fwd"] = {"ms": ms, "tflops": tf, "sclk_mhz": mhz, "socket_power_w": w}
    n = 8192
    g = torch.Generator(device="cpu").manual_seed(11)
    a = torch.randn(n, n, generator=g).to(torch.bfloat16).to(q.device)
    b = torch.randn(n, n, generator=g).to(torch.bfloat16).to(q.device)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=q.device)
    ms_g, mhz_g, w_g = sustained(torch, lambda: torch.matmul(a, b, out=c), 4.0, stream)
    tf_g = 2.0 * n ** 3 / ms_g / 1e9
    out["gemm_bf16"] = {"m_n_k": [n, n, n], "ms": ms_g, "tflops": tf_g, "frac_of_peak": tf_g / peak,
                        "sclk_mhz": mhz_g, "socket_power_w": w_g}
    out["fwd_frac_of_gemm"] = tf / tf_g
    if mhz:
        out["fwd_frac_of_peak_at_sclk"] = tf / (peak * mhz / 2400.0)
    del a, b, c
    # the same for e4m3 operands (torch._scaled_mm, bf16 out): the rate the
    # fp8 forward's row is compared with
    try:
        a8 = torch.randn(n, n, generator=g).to(q.device).to(torch.float8_e4m3fn)
        b8 = torch.randn(n, n, generator=g).to(q.device).to(torch.float8_e4m3fn).t()
        one = torch.ones((), device=q.device)
        ms_8, mhz_8, w_8 = sustained(
            torch, lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16), 4.0, stream)
        tf_8 = 2.0 * n ** 3 / ms_8 / 1e9
        out["gemm_fp8"] = {"m_n_k": [n, n, n], "ms": ms_8, "tflops": tf_8, "frac_of_fp8_peak": tf_8 / PEAK_TFLOPS["fp8"],
                           "sclk_mhz": mhz_8, "socket_power_w": w_8}
        del a8, b8
    except Exception as e:  # no fp8 GEMM in this torch build: the row keeps only its peak fraction
        out["gemm_fp8"] = {"error": repr(e)[:200]}
    return out


TOL_O = {"fp16": 2e-3, "bf16": 1.6e-2}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
CONFIG_COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_configs.json")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1)
    except Exception:
        return None


def config_counters(key):
    """MFMA busy share and HBM bytes of one workload's kernels, from the
    committed rocprofv3 counter summary, only if it was taken on the current
    kernel sources (else None)."""
    try:
        with open(CONFIG_COUNTERS_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("configs", {}).get(key)


def parity_fwd(o, lse, ro, rl, dtype, layout):
    import numpy as np

    from attn_inputs import to_bhsd64

    eo = float(np.abs(to_bhsd64(o.cpu(), layout) - ro).max())
    el = float(np.abs(lse.cpu().double().numpy() - rl).max())
    return {"o_maxabs": eo, "lse_maxabs": el, "tol_o": TOL_O[dtype], "tol_lse": TOL_LSE,
            "pass": bool(eo <= TOL_O[dtype] and el <= TOL_LSE)}


def parity_bwd(grads, refs, layout):
    import numpy as np

    from attn_inputs import to_bhsd64

    out = {}
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        out[name + "_relF"] = float(np.linalg.norm(to_bhsd64(g.cpu(), layout) - r) / np.linalg.norm(r))
    out["tol_relF"] = TOL_GRAD
    out["pass"] = bool(max(out[n + "_relF"] for n in ("dq", "dk", "dv")) <= TOL_GRAD)
    return out


def config_report(fa, torch, stream, peak_of, with_oracle=True, sustain_s=2.0):
    """The four smaller workloads (the 16K one is the step above), one entry
    per configuration and pass.  They run in microseconds, less than the
    Python binding takes to launch them, so each is timed two ways: 20
    launches captured in a HIP graph and replayed (GPU time per launch, no
    host gaps: the median of five batches of four replays, after three warm
    ones), and 100 launches from Python back to back (what
    an eager caller sees).  The graph is then replayed back to back for
    ``sustain_s`` seconds while amd-smi reads the GFX clock, which gives the
    fraction of the MFMA peak at the clock the part actually ran.  Parity:
    the same seeded inputs through the fp64 oracle (test infrastructure,
    timed on the host cores) against the GPU outputs, with the parity
    tests' tolerances.  MFMA busy and HBM GB/s come from the committed
    counter summary of these launches when it matches the kernel sources.
    With at most 512 workgroups they are occupancy- and latency-bound;
    their fraction of peak is context, not a target."""
    from attn_inputs import WORKLOADS, make_qkv, to_bhsd64

    def graph_of(fn):
        side = torch.cuda.Stream(device=stream.device)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(3):
                fn(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for _ in range(20):
                fn(cap)
        g.replay()
        torch.cuda.synchronize()
        return g

    def graph_ms(g):
        # warm replays first, then the median of five batches of four
        # replays (80 launches each), so that one slow batch (a clock
        # change, another process) does not set the figure
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(4):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / 80)
        return sorted(per)[2]

    def eager_ms(fn):
        for _ in range(10):
            fn(stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(100):
            fn(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 100

    def timed(fn, flop, peak, key):
        g = graph_of(fn)
        gm, em = graph_ms(g), eager_ms(fn)
        r = {"graph_ms": gm, "eager_loop_ms": em, "tflops": flop / gm / 1e9, "frac_of_peak": flop / gm / 1e9 / peak,
             "flop": flop}
        if sustain_s > 0:
            ms, mhz, w = sustained(torch, lambda: g.replay(), sustain_s, stream)
            r["sustained_ms"] = ms / 20
            r["sclk_mhz"], r["socket_power_w"] = mhz, w
            if mhz:
                r["frac_of_peak_at_sclk"] = flop / (ms / 20) / 1e9 / (peak * mhz / 2400.0)
        c = config_counters(key)
        if c is not None:
            r["mfma_busy"] = c.get("mfma_busy")
            if c.get("hbm_bytes") is not None:
                r["hbm_bytes"] = c["hbm_bytes"]
                r["hbm_gbs"] = c["hbm_bytes"] / (gm * 1e-3) / 1e9
        return r

    out = {}
    cores = blas_threads()
    for name, w in WORKLOADS.items():
        if w.N >= 16384:
            continue
        inp = make_qkv(w.B, w.H, w.N, w.N, w.d, w.dtype, w.layout, seed=w.seed, in_scale=w.in_scale,
                       with_do=w.backward)
        q, k, v = (inp[x].to(stream.device) for x in ("q", "k", "v"))
        s = 1.0 / math.sqrt(w.d)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
        peak = peak_of(w.dtype)
        for causal in w.causal:
            flop = 4.0 * w.B * w.H * w.N * w.N * w.d / (2 if causal else 1)
            # the key-split forward with its workspace (plain fa_fwd_ex kernels where it needs none)
            nws = fa.fa_fwd_splitk_workspace_bytes(w.B, w.H, w.N, w.N, w.d, causal)
            fws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
            fwd = lambda st: fa.fa_fwd_splitk(q, k, v, o, lse, s, causal, fws, (-1, -1), w.layout, st)
            key = "%s%s fwd" % (name, "" if len(w.causal) == 1 else (" causal" if causal else " noncausal"))
            out[key] = timed(fwd, flop, peak, key)
            out[key]["workload"] = "B%d H%d N%d d%d %s %s %s" % (w.B, w.H, w.N, w.d, w.dtype, w.layout.upper(),
                                                                  "causal" if causal else "non-causal")
            if w.backward:
                do = inp["do"].to(q.device)
                dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                # the workspace that lets an under-filled grid split its dK/dV stage
                ws = torch.empty(fa.fa_bwd_ex_workspace_bytes(w.B, w.H, w.H, w.N, w.N, w.d,
                                                              fa.FA_FP16 if w.dtype == "fp16" else fa.FA_BF16),
                                 dtype=torch.uint8, device=q.device)
                bwd = lambda st: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, st)
                out[name + " bwd"] = timed(bwd, 2.5 * flop, peak, name + " bwd")
                out[name + " bwd"]["workload"] = out[key]["workload"] + " backward"
            if with_oracle:
                from oracle import attention_bwd64, attention_fwd64

                fwd(stream)
                args = [to_bhsd64(inp[x], w.layout) for x in ("q", "k", "v")]
                t0 = time.perf_counter()
                ro, rl = attention_fwd64(*args, s, causal)
                t_o = time.perf_counter() - t0
                out[key]["parity"] = parity_fwd(o, lse, ro, rl, w.dtype, w.layout)
                out[key]["oracle"] = {"seconds": t_o, "gflops": flop / t_o / 1e9, "cores": cores}
                if w.backward:
                    bwd(stream)
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    refs = attention_bwd64(*args, to_bhsd64(inp["do"], w.layout), s, causal)
                    t_b = time.perf_counter() - t0
                    out[name + " bwd"]["parity"] = parity_bwd((dq, dk, dv), refs, w.layout)
                    out[name + " bwd"]["oracle"] = {"seconds": t_b, "gflops": 2.5 * flop / t_b / 1e9, "cores": cores}
    for kk, r in out.items():
        par = r.get("parity", {}).get("pass")
        log("  %-52s graph %.4f ms, eager %.4f ms, %.1f TFLOP/s (%.1f%% of peak%s), parity %s" % (
            kk, r["graph_ms"], r["eager_loop_ms"], r["tflops"], 100 * r["frac_of_peak"],
            ", %.1f%% at %.0f MHz" % (100 * r["frac_of_peak_at_sclk"], r["sclk_mhz"]) if r.get("sclk_mhz") else "",
            "pass" if par else ("FAIL" if par is not None else "n/a")))
    return out


def profile_configs(fa, torch, stream):
    """Launch each configuration's kernels a few times, eagerly and in a
    fixed order (the 16K step is left out), for a counter profile of this
    command: the report's MFMA busy and HBM figures come from such a run."""
    from attn_inputs import WORKLOADS, make_qkv

    order = []
    for name, w in WORKLOADS.items():
        if w.N >= 16384:
            continue
        inp = make_qkv(w.B, w.H, w.N, w.N, w.d, w.dtype, w.layout, seed=w.seed, in_scale=w.in_scale,
                       with_do=w.backward)
        q, k, v = (inp[x].to(stream.device) for x in ("q", "k", "v"))
        s = 1.0 / math.sqrt(w.d)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
        for causal in w.causal:
            key = "%s%s fwd" % (name, "" if len(w.causal) == 1 else (" causal" if causal else " noncausal"))
            nws = fa.fa_fwd_splitk_workspace_bytes(w.B, w.H, w.N, w.N, w.d, causal)
            fws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
            for _ in range(5):
                fa.fa_fwd_splitk(q, k, v, o, lse, s, causal, fws, (-1, -1), w.layout, stream)
            torch.cuda.synchronize()
            order.append(key)
            if w.backward:
                do = inp["do"].to(q.device)
                dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                ws = torch.empty(fa.fa_bwd_ex_workspace_bytes(w.B, w.H, w.H, w.N, w.N, w.d, fa.FA_FP16),
                                 dtype=torch.uint8, device=q.device)
                for _ in range(5):
                    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, stream)
                torch.cuda.synchronize()
                order.append(name + " bwd")
    # the fp8 forward of the 16K workload (its inputs cast to e4m3fn)
    w = WORKLOADS[WORKLOAD]
    inp = make_qkv(w.B, w.H, w.N, w.N, w.d, w.dtype, w.layout, seed=w.seed, in_scale=w.in_scale)
    q8, k8, v8 = (inp[x].to(stream.device).to(torch.float8_e4m3fn) for x in ("q", "k", "v"))
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q8.device)
    for _ in range(5):
        fa.fa_fwd_fp8(q8, k8, v8, o, lse, 1.0 / math.sqrt(w.d), True, (-1, -1), (1.0, 1.0, 1.0), "bhsd", stream)
    torch.cuda.synchronize()
    order.append("fp8_fwd")
    return order


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only
    if it was taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


CPU_SAMPLE_HEADS = 4


def cpu_baseline(inp, s, causal, gpu_out):
    """fp64 oracle on the first CPU_SAMPLE_HEADS heads of batch 0: forward +
    backward, wall-clock timed (a bounded sample of the same workload)."""
    import numpy as np

    from attn_inputs import to_bhsd64
    from oracle import attention_bwd64, attention_fwd64

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max((p.get("num_threads", 1) for p in threadpool_info()
                            if p.get("user_api") == "blas"), default=1)
    except Exception:
        blas_threads = None
    nh = CPU_SAMPLE_HEADS
    q, k, v, do = (to_bhsd64(inp[x][:1, :nh]) for x in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    o, lse = attention_fwd64(q, k, v, s, causal)
    dq, dk, dv = attention_bwd64(q, k, v, do, s, causal)
    dt = time.perf_counter() - t0
    N, d = q.shape[2], q.shape[3]
    flop = nh * 4.0 * N * N * d / (2 if causal else 1) * 3.5
    # the GPU result for the same heads, as a by-product check
    go, glse, gdq, gdk, gdv = gpu_out
    err_o = float(np.abs(to_bhsd64(go[:1, :nh]) - o).max())
    err_l = float(np.abs(glse[:1, :nh].double().numpy() - lse).max())
    rel = [float(np.linalg.norm(to_bhsd64(g[:1, :nh]) - r) / np.linalg.norm(r))
           for g, r in ((gdq, dq), (gdk, dk), (gdv, dv))]
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads,
        "kind": "oracle",
        "sample": "fp64 numpy oracle, forward + backward of %d of 16 heads (b=0, h=0..%d) of the same "
                  "workload; %.1f s wall; BLAS threads %s, elementwise numpy single-threaded; host cores visible %d"
                  % (nh, nh - 1, dt, blas_threads, len(os.sched_getaffinity(0))),
        "seconds": dt,
        "parity_sampled_heads": {"o_maxabs": err_o, "lse_maxabs": err_l, "dq_relF": rel[0], "dk_relF": rel[1],
                         "dv_relF": rel[2]},
    }


C4_SAMPLE_ROWS = 256


def c4_sampled_parity(inp, o, lse, s, w):
    """The 16K forward on C4_SAMPLE_ROWS seeded query rows of every head
    (rows 0 and N-1 always) against the oracle, as the parity tests check it."""
    import numpy as np

    from attn_inputs import sample_rows, to_bhsd64
    from oracle import attention_rows_fwd64

    rows = sample_rows(w.B, w.H, w.N, C4_SAMPLE_ROWS, w.seed + 1000)
    q, k, v = (to_bhsd64(inp[x]) for x in ("q", "k", "v"))
    t0 = time.perf_counter()
    ro, rl = attention_rows_fwd64(q, k, v, s, True, rows)
    dt = time.perf_counter() - t0
    og, lg = to_bhsd64(o.cpu()), lse.cpu().double().numpy()
    go = np.stack([np.stack([og[b, h][rows[b, h]] for h in range(w.H)]) for b in range(w.B)])
    gl = np.stack([np.stack([lg[b, h][rows[b, h]] for h in range(w.H)]) for b in range(w.B)])
    eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
    flop = 4.0 * w.d * float(sum(int(r) + 1 for r in rows.ravel()))
    full = 4.0 * w.B * w.H * w.N * w.N * w.d / 2  # the whole causal forward
    return {"rows_per_head": int(rows.shape[2]), "o_maxabs": eo, "lse_maxabs": el, "tol_o": TOL_O[w.dtype],
            "tol_lse": TOL_LSE, "pass": bool(eo <= TOL_O[w.dtype] and el <= TOL_LSE),
            "oracle": {"seconds": dt, "gflops": flop / dt / 1e9, "cores": blas_threads(),
                       "extrapolated_full_forward_seconds": dt * full / flop,
                       "note": "extrapolated: the sampled rows' time scaled by the whole forward's FLOP "
                               "over the sampled rows' FLOP"}}


def noncausal_row(fa, torch, q, k, v, do, s, stream, peak, steps, with_oracle=True):
    """A chip-filling non-causal row: the 16K inputs without the causal
    mask (2048 forward workgroups), forward and backward, timed with HIP
    events; forward parity on 64 seeded rows per head."""
    import numpy as np

    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_BF16), dtype=torch.uint8, device=q.device)
    for _ in range(2):
        fa.fa_fwd(q, k, v, o, lse, s, False, stream)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, s, False, ws, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tf = tb = 0.0
    for _ in range(steps):
        ev[0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, s, False, stream)
        ev[1].record(stream)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, s, False, ws, stream)
        ev[2].record(stream)
        torch.cuda.synchronize()
        tf += ev[0].elapsed_time(ev[1])
        tb += ev[1].elapsed_time(ev[2])
    tf, tb = tf / steps, tb / steps
    ff = 4.0 * B * H * N * N * d
    key = "fwd_b1h16_n16384_d128_bf16_bhsd noncausal"
    r = {"workload": "B1 H16 N16384 d128 bf16 BHSD non-causal (the 16K inputs)", "fwd_ms": tf,
         "fwd_tflops": ff / tf / 1e9, "fwd_frac_of_peak": ff / tf / 1e9 / peak, "bwd_ms": tb,
         "bwd_tflops": 2.5 * ff / tb / 1e9, "bwd_frac_of_peak": 2.5 * ff / tb / 1e9 / peak}
    log("  %-52s fwd %.3f ms (%.1f TFLOP/s, %.1f%%), bwd %.3f ms (%.1f TFLOP/s)" % (
        key, tf, ff / tf / 1e9, 100 * ff / tf / 1e9 / peak, tb, 2.5 * ff / tb / 1e9))
    if with_oracle:
        from attn_inputs import sample_rows, to_bhsd64
        from oracle import attention_rows_fwd64

        rows = sample_rows(B, H, N, 64, 7)
        qc, kc, vc = (to_bhsd64(x.cpu()) for x in (q, k, v))
        t0 = time.perf_counter()
        ro, rl = attention_rows_fwd64(qc, kc, vc, s, False, rows)
        dt = time.perf_counter() - t0
        og, lg = to_bhsd64(o.cpu()), lse.cpu().double().numpy()
        go = np.stack([np.stack([og[b, h][rows[b, h]] for h in range(H)]) for b in range(B)])
        gl = np.stack([np.stack([lg[b, h][rows[b, h]] for h in range(H)]) for b in range(B)])
        eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
        r["parity_fwd_sampled_rows"] = {"rows_per_head": 64, "o_maxabs": eo, "lse_maxabs": el,
                                        "pass": bool(eo <= TOL_O["bf16"] and el <= TOL_LSE),
                                        "oracle": {"seconds": dt, "gflops": 4.0 * d * N * rows.size / dt / 1e9,
                                                   "cores": blas_threads()}}
    return {key + "+bwd": r}


GQA_KV_HEADS = 2          # 16 query heads on 2 K/V heads (G = 8)
WINDOW = (256, 256)       # the skill guide's sliding-window example, with causal
DROPOUT = (0.1, 2024, 0)  # the skill guide's dropout_p = 0.1 (seed, offset arbitrary)


def next_rows(fa, torch, q, k, v, do, s, stream, peak, steps):
    """Forward + backward of the built 'next' rows on the same 16K inputs:
    fewer K/V heads (the first GQA_KV_HEADS heads of k, v shared by all 16
    query heads, causal), a causal sliding window WINDOW, and causal dropout
    DROPOUT; and the fp8 forward (forward only) on the inputs cast to
    float8_e4m3fn, against the fp8 MFMA peak.  FLOPs count the admitted
    (query, key) pairs; the backward is 2.5x the forward."""
    B, H, N, d = q.shape
    res = {}
    kg, vg = k[:, :GQA_KV_HEADS].contiguous(), v[:, :GQA_KV_HEADS].contiguous()
    pairs_causal = N * (N + 1) / 2
    lft = WINDOW[0]
    pairs_win = sum(min(i, lft) + 1 for i in range(N))
    cases = {
        "gqa": dict(k=kg, v=vg, window=(-1, -1), pairs=pairs_causal, dropout=None,
                    desc="B1 H16 H_kv%d N16384 d128 bf16 causal" % GQA_KV_HEADS),
        "sliding_window": dict(k=k, v=v, window=WINDOW, pairs=pairs_win, dropout=None,
                               desc="B1 H16 N16384 d128 bf16 causal, window %r" % (WINDOW,)),
        "dropout": dict(k=k, v=v, window=(-1, -1), pairs=pairs_causal, dropout=DROPOUT,
                        desc="B1 H16 N16384 d128 bf16 causal, dropout_p %g" % DROPOUT[0]),
        # one GPU's share if the 16 heads were split over 8 GPUs (no exchange
        # is needed between them): the same kernels on 2 heads
        "head_shard_8": dict(q=q[:, :2].contiguous(), do=do[:, :2].contiguous(), k=k[:, :2].contiguous(),
                             v=v[:, :2].contiguous(), window=(-1, -1), pairs=pairs_causal, dropout=None,
                             desc="B1 H2 N16384 d128 bf16 causal (2 of the 16 heads: one GPU of 8 under head "
                                  "sharding)"),
    }
    for name, c in cases.items():
        qc, dc = c.get("q", q), c.get("do", do)
        Hc = qc.shape[1]
        o = torch.empty_like(qc)
        lse = torch.empty((B, Hc, N), dtype=torch.float32, device=q.device)
        dq, dk, dv = torch.empty_like(qc), torch.empty_like(c["k"]), torch.empty_like(c["v"])
        # with fewer K/V heads, the workspace that lets the dK/dV stage split
        ws = torch.empty(fa.fa_bwd_ex_workspace_bytes(B, Hc, c["k"].shape[1], N, N, d, fa.FA_BF16), dtype=torch.uint8,
                         device=q.device)

        # the key-split forward where the grid is too small for the chip (the head-shard row)
        nws = fa.fa_fwd_splitk_workspace_bytes(B, Hc, N, N, d, True, c["window"])
        fws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None

        def fwd():
            fa.fa_fwd_splitk(qc, c["k"], c["v"], o, lse, s, True, fws, c["window"], "bhsd", stream, c["dropout"])

        def bwd():
            fa.fa_bwd_ex(qc, c["k"], c["v"], o, lse, dc, dq, dk, dv, s, True, ws, c["window"], fa.FA_BWD_ALL,
                         "bhsd", stream, c["dropout"])

        for _ in range(2):
            fwd()
            bwd()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        tf = tb = 0.0
        for _ in range(steps):
            ev[0].record(stream)
            fwd()
            ev[1].record(stream)
            bwd()
            ev[2].record(stream)
            torch.cuda.synchronize()
            tf += ev[0].elapsed_time(ev[1])
            tb += ev[1].elapsed_time(ev[2])
        tf, tb = tf / steps, tb / steps
        ff = 4.0 * B * Hc * d * c["pairs"]
        res[name] = {"workload": c["desc"], "fwd_ms": tf, "bwd_ms": tb,
                     "fwd_tflops": ff / tf / 1e9, "bwd_tflops": 2.5 * ff / tb / 1e9,
                     "step_tflops": 3.5 * ff / (tf + tb) / 1e9, "fwd_frac_of_peak": ff / tf / 1e9 / peak}
        log("%s: fwd %.3f ms (%.1f TFLOP/s), bwd %.3f ms (%.1f TFLOP/s)" % (
            name, tf, ff / tf / 1e9, tb, 2.5 * ff / tb / 1e9))

    q8, k8, v8 = (t.to(torch.float8_e4m3fn) for t in (q, k, v))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)

    def fwd8():
        fa.fa_fwd_fp8(q8, k8, v8, o, lse, s, True, (-1, -1), (1.0, 1.0, 1.0), "bhsd", stream)

    # a forward-only row is short: warm up for ~10 ms (clocks settle after
    # the heavier rows) and time at least 20 launches
    for _ in range(20):
        fwd8()
    n8 = max(steps, 20)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(n8):
        fwd8()
    ev[1].record(stream)
    torch.cuda.synchronize()
    tf = ev[0].elapsed_time(ev[1]) / n8
    ff = 4.0 * B * H * d * pairs_causal
    res["fp8_fwd"] = {"workload": "B1 H16 N16384 d128 float8_e4m3fn causal (the bf16 inputs cast), bf16 out",
                      "fwd_ms": tf, "fwd_tflops": ff / tf / 1e9, "peak": PEAK_TFLOPS["fp8"],
                      "fwd_frac_of_peak": ff / tf / 1e9 / PEAK_TFLOPS["fp8"],
                      "traffic": measured_traffic("fp8_fwd")}
    log("fp8_fwd: fwd %.3f ms (%.1f TFLOP/s, %.1f%% of the fp8 peak)" % (
        tf, ff / tf / 1e9, 100 * ff / tf / 1e9 / PEAK_TFLOPS["fp8"]))
    return res


def copy_calibration(torch, dev, mib):
    """A plain device copy of `mib` MiB, three times: a counter profile of
    the command reads FETCH_SIZE / WRITE_SIZE of known bytes from it."""
    if mib <= 0:
        return
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows-f", action="store_true",
                    help="skip the GQA / sliding-window measurements (profiles of the main step use this, "
                         "since those runs launch the same kernel instantiations)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (3 times), so a counter "
                         "profile of this command can calibrate FETCH_SIZE/WRITE_SIZE against known bytes")
    ap.add_argument("--no-power-context", action="store_true",
                    help="skip the clock/power readings and the GEMM comparison")
    ap.add_argument("--no-small-configs", action="store_true",
                    help="skip the report on the four smaller workloads and the non-causal row")
    ap.add_argument("--no-oracle", action="store_true",
                    help="skip every oracle computation (parity entries of the report, cpu_baseline)")
    ap.add_argument("--profile-configs", action="store_true",
                    help="only launch each smaller workload's kernels 5 times in a fixed order (for a counter "
                         "profile of this command) and print that order")
    args = ap.parse_args()
    if args.no_oracle:
        args.no_cpu_baseline = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(attention heads shard with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_io_aware_02_amd as fa
    from attn_inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[WORKLOAD]
    causal = True
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_configs:
        copy_calibration(torch, dev, args.copy_calibration_mib)
        order = profile_configs(fa, torch, torch.cuda.current_stream(dev))
        print(json.dumps({"profile_configs_order": order}), flush=True)
        return
    inp = workload_inputs(w)
    rng = np.random.default_rng(w.seed + 2000)
    inp["do"] = torch.from_numpy(rng.standard_normal(inp["q"].shape, dtype=np.float32)).to(torch.bfloat16)
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    s = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d, fa.FA_BF16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.fa_fwd(q, k, v, o, lse, s, causal, stream)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, stream)

    copy_calibration(torch, dev, args.copy_calibration_mib)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, s, causal, stream)
        ev[i][1].record(stream)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    step_ms = ev[0][0].elapsed_time(ev[-1][2]) / K
    ms_per_step = max(step_ms, wall * 1e3 / K)

    # each backward stage alone, same stream, K launches
    stage_ms = {}
    for name, flag in (("bwd_prep", fa.FA_BWD_PREP), ("bwd_dkdv", fa.FA_BWD_DKDV), ("bwd_dq", fa.FA_BWD_DQ)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fa.fa_bwd_stages(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, flag, "bhsd", stream)
        e0.record(stream)
        for _ in range(K):
            fa.fa_bwd_stages(q, k, v, o, lse, do, dq, dk, dv, s, causal, ws, flag, "bhsd", stream)
        e1.record(stream)
        torch.cuda.synchronize()
        stage_ms[name] = e0.elapsed_time(e1) / K

    fwd_flop = 4.0 * B * H * N * N * d / (2 if causal else 1)
    bwd_flop = 2.5 * fwd_flop
    value = (fwd_flop + bwd_flop) / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    # algorithmic work per launch of each kernel: the backward's five
    # contractions (S recompute, dP, dV, dK, dQ) split four to dK/dV, one to dQ
    kernels = {
        "fwd": {"ms": fwd_ms, "flop": fwd_flop},
        "bwd_dkdv": {"ms": stage_ms["bwd_dkdv"], "flop": 2.0 * fwd_flop},
        "bwd_dq": {"ms": stage_ms["bwd_dq"], "flop": 0.5 * fwd_flop},
        "bwd_prep": {"ms": stage_ms["bwd_prep"], "bytes": B * H * N * (2 * d * 2 + 4)},
    }

    def roof(name):
        kk = kernels[name]
        tr = measured_traffic(name)
        gbs = None if tr is None else tr / (kk["ms"] * 1e-3) / 1e9  # measured HBM GB/s
        if "flop" in kk:
            ach = kk["flop"] / (kk["ms"] * 1e-3) / 1e12
            return {"kernel": name, "bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                    "frac": ach / peak, "traffic": tr, "traffic_gbs": gbs, "ms_per_launch": kk["ms"],
                    "algorithmic_flop_per_launch": kk["flop"]}
        ach = kk["bytes"] / (kk["ms"] * 1e-3) / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "traffic": tr, "traffic_gbs": gbs, "ms_per_launch": kk["ms"],
                "algorithmic_bytes_per_launch": kk["bytes"]}

    dominant = max(kernels, key=lambda n: kernels[n]["ms"])
    log("step %.3f ms  (fwd %.3f ms, bwd %.3f ms: prep %.3f dkdv %.3f dq %.3f)" % (
        ms_per_step, fwd_ms, bwd_ms, stage_ms["bwd_prep"], stage_ms["bwd_dkdv"], stage_ms["bwd_dq"]))
    log("fwd %.1f TFLOP/s (%.1f%% of %.0f), bwd %.1f TFLOP/s, step %.1f TFLOP/s" % (
        fwd_flop / fwd_ms / 1e9, 100 * fwd_flop / fwd_ms / 1e9 / peak, peak, bwd_flop / bwd_ms / 1e9, value))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1) x0.5 inputs, iid N(0,1) dO)",
        "config": {"workload": WORKLOAD + " forward+backward", "B": B, "H": H, "Nq": N, "Nk": N, "d": d,
                   "causal": causal, "layout": "bhsd", "scale": s},
        "frac_of_peak": value / peak,
        "fwd": {"ms": fwd_ms, "tflops": fwd_flop / fwd_ms / 1e9, "frac_of_peak": fwd_flop / fwd_ms / 1e9 / peak},
        "bwd": {"ms": bwd_ms, "tflops": bwd_flop / bwd_ms / 1e9, "frac_of_peak": bwd_flop / bwd_ms / 1e9 / peak,
                "stages_ms": stage_ms},
        "roofline": roof(dominant),
        "roofline_fwd": roof("fwd"),
    }
    if not args.no_power_context:
        out["power_context"] = power_context(torch, fa, q, k, v, o, lse, s, causal, stream, fwd_flop, peak)
        pc = out["power_context"]
        log("power context: fwd %.1f TFLOP/s at %s MHz / %s W; bf16 GEMM 8192^3 %.1f TFLOP/s at %s MHz / %s W" % (
            pc["fwd"]["tflops"], pc["fwd"]["sclk_mhz"], pc["fwd"]["socket_power_w"], pc["gemm_bf16"]["tflops"],
            pc["gemm_bf16"]["sclk_mhz"], pc["gemm_bf16"]["socket_power_w"]))
        if pc["gemm_fp8"].get("tflops"):
            log("power context: fp8 GEMM 8192^3 %.1f TFLOP/s at %s MHz / %s W" % (
                pc["gemm_fp8"]["tflops"], pc["gemm_fp8"]["sclk_mhz"], pc["gemm_fp8"]["socket_power_w"]))
    if not args.no_small_configs:
        log("configurations:")
        out["configs"] = config_report(fa, torch, stream, lambda dt: PEAK_TFLOPS[dt], with_oracle=not args.no_oracle)
        nc = noncausal_row(fa, torch, q, k, v, do, s, stream, peak, min(K, 10), with_oracle=not args.no_oracle)
        out["configs"].update(nc)
    if not args.no_rows_f:
        out["rows_f"] = next_rows(fa, torch, q, k, v, do, s, stream, peak, min(K, 10))
        g8 = (out.get("power_context") or {}).get("gemm_fp8") or {}
        if g8.get("tflops"):
            r8 = out["rows_f"]["fp8_fwd"]
            r8["frac_of_fp8_gemm"] = r8["fwd_tflops"] / g8["tflops"]
            log("fp8_fwd: %.1f%% of the fp8 GEMM's %.1f TFLOP/s under the same cap" % (
                100 * r8["frac_of_fp8_gemm"], g8["tflops"]))
    # the 16K workload's entry of the per-configuration report
    c4 = {"workload": "B1 H16 N16384 d128 bf16 BHSD causal, inputs x0.5",
          "fwd_ms": fwd_ms, "fwd_tflops": fwd_flop / fwd_ms / 1e9, "fwd_frac_of_peak": fwd_flop / fwd_ms / 1e9 / peak,
          "bwd_ms": bwd_ms, "bwd_tflops": bwd_flop / bwd_ms / 1e9, "bwd_frac_of_peak": bwd_flop / bwd_ms / 1e9 / peak}
    pc = out.get("power_context")
    if pc and pc["fwd"].get("sclk_mhz"):
        c4["fwd_sclk_mhz"] = pc["fwd"]["sclk_mhz"]
        c4["fwd_frac_of_peak_at_sclk"] = pc["fwd_frac_of_peak_at_sclk"]
    cnt = config_counters(WORKLOAD)
    if cnt is not None:
        c4["counters"] = cnt
    if not args.no_oracle:
        c4["parity_fwd_sampled_rows"] = c4_sampled_parity(inp, o, lse, s, w)
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        gpu_out = (o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu())
        out["cpu_baseline"] = cpu_baseline(inp, s, causal, gpu_out)
        ph = out["cpu_baseline"]["parity_sampled_heads"]
        c4["parity_heads_0_3"] = dict(ph, **{"pass": bool(
            ph["o_maxabs"] <= TOL_O[w.dtype] and ph["lse_maxabs"] <= TOL_LSE
            and max(ph["dq_relF"], ph["dk_relF"], ph["dv_relF"]) <= TOL_GRAD)})
        log("cpu_baseline: %.4f TFLOP/s over %.1f s; sampled-head parity %s" % (
            out["cpu_baseline"]["value"], out["cpu_baseline"]["seconds"], out["cpu_baseline"]["parity_sampled_heads"]))
    out.setdefault("configs", {})[WORKLOAD + " fwd+bwd"] = c4
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
