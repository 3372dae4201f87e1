#!/usr/bin/env python3
"""Throughput of the GPT-2 training step on one MI355X.

Workload (default): GPT-2 124M (L=12, NH=12, C=768, V=50257 padded to
50304), bf16 activations and matrix products with fp32 master weights,
gradients and AdamW state; micro-batch B=8, T=1024; one step = 2 micro-steps
(forward + backward, gradients accumulated with dloss = 1/(2*B*T)) + one AdamW
update (lr 6e-4, betas 0.9/0.999, eps 1e-8, weight decay 0.1).  Random GPT-2
initialisation and a Zipf(1.1) token stream (seeded, synthetic), all resident
in HBM before the timed region.

Prints one JSON line: train tokens/s over the timed steps, MFU against the
2.5 PFLOP/s dense bf16 peak, the roofline position of the dominant kernel
(the grouped launches of every weight gradient of a micro-step, timed with
HIP events that the library records around them inside the timed steps, on
the step's stream), the
position of every kernel family from two further instrumented steps, and the
CPU oracle timed on a bounded sample of the same workload.

Other workloads: --model 1558m (GPT-2 1.5B, 10 steps of B=8 T=1024, lr 3e-4,
wd 0, no accumulation, peak HBM reported), --workload c2 (GPT-2 124M fp32,
B=4 T=64, 10 AdamW steps on one batch, lr 1e-4), --workload fused (the
standalone fp32 Linear+GELU+softmax op), --workload generate (the page's
generation loop).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def flops_per_token(L, C, V, T):
    """Algorithmic training FLOPs per token: 3x the forward's
    24 L C^2 (layer products) + 2 C V (classifier over the real vocabulary)
    + 2 L (T+1) C (causal attention scores and weighted sum)."""
    return 3.0 * (24.0 * L * C * C + 2.0 * C * V + 2.0 * L * (T + 1) * C)


def host_cpu():
    """The host's CPU model and logical core count."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline(cfg, T=256, name="124M", bf16_init=True):
    """The CPU oracle (single-threaded C, fp64) on a bounded sample of the same
    workload: one micro-step (forward + backward) of the model on B=1 x T
    tokens, about 30 s on the host cores for 124M at T = 256 (T = 1024 would
    take about 2 minutes; per-token work at T = 256 is within 8% of it, the
    causal attention's share being the difference)."""
    import oracle
    import synthetic as S
    params = S.init_params(cfg)
    if bf16_init:
        params = {k: S.round_to_bf16(v) for k, v in params.items()}
    flat = oracle.pack_params(cfg, params)
    stream = S.token_stream(T + 1, cfg.vocab_size, dist="zipf")
    x, y = S.batch(stream, 0, 1, T)
    t0 = time.perf_counter()
    oracle.gpt2_step(cfg, flat, x, y)
    dt = time.perf_counter() - t0
    model, ncpu = host_cpu()
    return {"value": round(T / dt, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"one forward+backward micro-step of GPT-2 {name}, B=1 T={T} (fp64, single thread), "
                      f"{dt:.1f} s",
            "host_cpu": model, "host_nproc": ncpu}


PEAK_FP32_TFLOPS = 157.3


def bench_fused(args):
    """The standalone fp32 op Y = softmax_row(GELU_tanh(X W^T + b)), X [1024,8192],
    W [8192,8192]: median time per call of `steps` calls after `warmup`."""
    import torch
    import synthetic as S
    from transformer_lm_step_amd import binding as Bnd

    M, K, N = 1024, 8192, 8192
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    X, W, b = S.fused_op_inputs(M, K, N)
    x, w, bb = (torch.from_numpy(a).to(dev) for a in (X, W, b))
    y = torch.empty(M, N, dtype=torch.float32, device=dev)
    wsz = Bnd.fused_linear_gelu_softmax_f32_workspace(M, N)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    cur = torch.cuda.current_stream()
    sh = cur.cuda_stream

    def call():
        Bnd.fused_linear_gelu_softmax_f32(x.data_ptr(), w.data_ptr(), bb.data_ptr(), y.data_ptr(), M, K, N,
                                          ws.data_ptr(), wsz, sh)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        call()
        e1.record(cur)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(c) for a, c in times]))
    flop = 2.0 * M * N * K
    tf = flop / (ms / 1e3) / 1e12
    rows_sum = y.sum(1)
    if not bool(torch.all((rows_sum - 1).abs() < 1e-4)):
        raise RuntimeError("fused op: rows do not sum to 1")
    log(f"bench: fused op {ms:.3f} ms/call, {tf:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = np.arange(16, dtype=np.int32)
        t0 = time.perf_counter()
        oracle.fused_linear_gelu_softmax(X, W, b, rows=rows)
        dt = time.perf_counter() - t0
        cpu = {"value": round(dt * M / rows.size * 1e3, 1), "unit": "ms/call", "cores": 1, "kind": "oracle",
               "sample": f"16 of the 1024 rows (fp64, single thread) in {dt:.1f} s, scaled to 1024 rows"}
    out = {
        "metric": "ms per call, fused Linear+GELU_tanh+row softmax fp32",
        "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "strong", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (X ~ N(0,1), W ~ N(0,1/8192), b ~ N(0,0.02))",
        "config": {"workload": "fused Linear+GELU+softmax, X[1024,8192] W[8192,8192] b[8192]"},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP32_TFLOPS, 4), "traffic": None,
                     "kernel": "gemm_kernel + softmax_finish_kernel (whole call)", "avg_ms": round(ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_generate(args):
    """The page's generation loop on GPT-2 124M bf16 (B=8, T=1024): per new
    token a forward without targets over all B x T positions, then one draw
    per batch row on the device (gpt2_generate).  `steps` tokens per row are
    generated after `warmup` untimed ones; value = generated tokens/s over all
    rows.  The classifier product is again the dominant kernel (HIP events
    around its launches in the timed forwards)."""
    import torch
    import synthetic as S
    from transformer_lm_step_amd import binding as Bnd
    from transformer_lm_step_amd.model import GPT2

    cfg = S.GPT2_124M
    B, T = args.batch, args.seq
    if args.warmup + args.steps >= T:
        raise SystemExit("generate: warmup + steps must stay below the sequence length")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = GPT2(cfg, Bnd.GPT2_BF16, B, T)
    model.init(model.pack({k: S.round_to_bf16(v) for k, v in S.init_params(cfg).items()}))
    rng = np.random.default_rng(12)
    t_begin = T - args.warmup - args.steps
    start = S.token_stream(B * T, cfg.vocab_size, dist="zipf").reshape(B, T)
    tok = torch.from_numpy(start.copy()).to(dev)
    coins = torch.from_numpy(rng.random((args.warmup + args.steps) * B).astype(np.float32)).to(dev)
    t_mid = t_begin + args.warmup
    model.generate(tok, coins, t_begin, t_mid)
    torch.cuda.synchronize()
    hip = HipEvents()
    starts, ends = hip.create(args.steps), hip.create(args.steps)
    hook = Bnd.gpt2_set_classifier_events(model.ctx, starts, ends)
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    model.generate(tok, coins[args.warmup * B:], t_mid, T)
    e1.record(cur)
    torch.cuda.synchronize()
    Bnd.gpt2_set_classifier_events(model.ctx, [], [])
    del hook
    if model.check() != 0:
        raise RuntimeError("device-side error during generation")
    ms = e0.elapsed_time(e1) / args.steps
    kms = float(np.mean([hip.elapsed_ms(a, b) for a, b in zip(starts, ends)]))
    hip.destroy(starts + ends)
    # the draw alone: the sampling kernel over the last forward's logits
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(cur)
    for _ in range(20):
        model.sample(coins[:B], tok, T - 1)
    s1.record(cur)
    torch.cuda.synchronize()
    sample_us = s0.elapsed_time(s1) / 20 * 1e3
    gen = tok.cpu().numpy()
    if not (np.all(gen >= 0) and np.all(gen < cfg.vocab_size)):
        raise RuntimeError("generated ids outside the vocabulary")
    tok_s = B / (ms / 1e3)
    kflop = 2.0 * B * T * cfg.padded_vocab_size * cfg.channels
    achieved = kflop / (kms / 1e3) / 1e12
    log(f"bench: generate {ms:.3f} ms per token step ({tok_s:,.0f} tok/s), classifier {kms:.3f} ms, "
        f"draw {sample_us:.1f} us")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        Tc, n = 64, 4
        flat = oracle.pack_params(cfg, {k: S.round_to_bf16(v) for k, v in S.init_params(cfg).items()})
        t0 = time.perf_counter()
        oracle.generate(cfg, flat, start[:1, :Tc], rng.random((n, 1)), Tc - n, Tc)
        dt = time.perf_counter() - t0
        cpu = {"value": round(n / dt, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} tokens of one row at T={Tc} (full forward per token, fp64, single thread), "
                         f"{dt:.1f} s"}
    out = {
        "metric": "generated tokens/s, GPT-2 124M bf16, full B x T forward per token (page's loop)",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (Zipf(1.1) prompt tokens, random GPT-2 init, uniform coins)",
        "config": {"workload": f"GPT-2 124M generation: B={B} rows, T={T}, one draw per row per forward"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "gemm_dtl_kernel (classifier forward, in the timed forwards)",
                     "avg_ms": round(kms, 4), "launches": args.steps},
        "sample_kernel_us": round(sample_us, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    model.close()


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (plumbing for the
    library's timing hook; torch creates its events lazily)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = self.ct.c_void_p()
            if self.rt.hipEventCreate(self.ct.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        if self.rt.hipEventSynchronize(b) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        t = self.ct.c_float()
        if self.rt.hipEventElapsedTime(self.ct.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)


HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(HERE, "transformer_lm_step_amd", "csrc", "gemm.hip")


def gemm_source_hash():
    import hashlib
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_probe():
    """Kernels for the HBM-traffic counter runs: a 1 GiB device copy (the
    reference of known size), 3 launches, then two steps of the benchmark
    workload (one warm-up, one whose dispatches the summaries read)."""
    import torch
    dev = torch.device("cuda:0")
    n = 1 << 28  # 2^28 floats = 1 GiB
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    args = argparse.Namespace(model="124m", batch=8, seq=1024, accum=2, steps=1, warmup=1, sr=False,
                              no_cpu_baseline=True)
    bench_gpt2(args)
    print(json.dumps({"traffic_probe": "done", "gemm_source_sha256": gemm_source_hash()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 10 for --model 1558m and --workload c2)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--seq", type=int, default=1024)
    ap.add_argument("--accum", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only launch the kernels the HBM-traffic counter runs read")
    ap.add_argument("--model", choices=("124m", "1558m"), default="124m",
                    help="GPT-2 size of the training step (124M is the headline workload)")
    ap.add_argument("--sr", action="store_true",
                    help="train without fp32 master weights (bf16 parameters, stochastic rounding in AdamW)")
    ap.add_argument("--profile-summary", nargs="+", metavar="DIR",
                    help="print markdown tables from rocprofv3 output folders of this bench (kernel stats of a "
                         "--kernel-trace --stats run; per-kernel means of --pmc runs) instead of running")
    ap.add_argument("--workload", choices=("gpt2", "c2", "fused", "generate"), default="gpt2",
                    help="gpt2: the GPT-2 training step (default); c2: GPT-2 124M fp32 at B=4 T=64; "
                         "fused: the standalone Linear+GELU+softmax op; generate: the page's generation loop")
    args = ap.parse_args()
    if args.steps is None and args.workload in ("fused", "generate"):
        args.steps = 20
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the data-parallel multi-GPU path is not implemented.", file=sys.stderr)
        sys.exit(2)
    if args.profile_summary:
        profile_summary(args.profile_summary)
        return
    if args.traffic_probe:
        traffic_probe()
        return
    if args.workload == "fused":
        bench_fused(args)
        return
    if args.workload == "generate":
        bench_generate(args)
        return
    if args.workload == "c2":
        bench_c2(args)
        return

    bench_gpt2(args)


# ---------------------------------------------------------------------------
# kernel families of the step: launch points of the library's timing hooks
# and the algorithmic work of each launch, in launch order per call

FAMILIES = [  # (name, timing point, bound)
    ("weight gradients (all layers + classifier, grouped launches)", "WEIGHT_GRAD", "mfma"),
    ("classifier forward", "CLASSIFIER_FWD", "mfma"),
    ("classifier input gradient", "CLASSIFIER_DX", "mfma"),
    ("layer forward products", "LAYER_FWD", "mfma"),
    ("layer input-gradient products", "LAYER_DX", "mfma"),
    ("attention forward", "ATTN_FWD", "mfma"),
    ("attention backward", "ATTN_BWD", "mfma"),
    ("LayerNorm forward", "LN_FWD", "hbm"),
    ("LayerNorm backward", "LN_BWD", "hbm"),
    ("softmax cross-entropy", "CE", "hbm"),
    ("token/position embedding backward", "ENCODER_BWD", "hbm"),
    ("AdamW", "ADAMW", "hbm"),
]


def _short_kernel_name(name):
    n = name.replace("(anonymous namespace)::", "").replace("void ", "").strip()
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):  # cut the argument list: the first "(" outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return n[:cut]


def _find(folder, suffix):
    hits = []
    for root, _, files in os.walk(folder):
        hits += [os.path.join(root, f) for f in files if f.endswith(suffix)]
    return sorted(hits)


def profile_summary(folders):
    """Markdown tables from rocprofv3 output folders of this bench.

    Kernel statistics (--kernel-trace --stats): per kernel, per optimizer step
    (the step count is the number of AdamW launches in the run).  Counter runs
    (--pmc over --traffic-probe): the per-dispatch mean of each counter per
    kernel, plus derived columns: HBM MB per dispatch from FETCH_SIZE and
    WRITE_SIZE (KiB, each scaled by what it reads for the probe's 1 GiB device
    copies) and, with a kernel-statistics folder among the arguments, GB/s
    over that kernel's average duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES
    / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); dependency wait =
    SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; LDS conflict = SQ_LDS_BANK_CONFLICT /
    SQ_LDS_IDX_ACTIVE; L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS) and the
    L2 request rate per XCD over the kernel's average duration."""
    import csv
    avg_us = {}
    counters = {}  # kernel -> {counter: (sum, n)}
    scale = {}
    for folder in folders:
        for path in _find(folder, "kernel_stats.csv"):
            rows = list(csv.DictReader(open(path)))
            steps = sum(int(r["Calls"]) for r in rows if "adamw" in r["Name"])
            tot = sum(float(r["TotalDurationNs"]) for r in rows)
            print(f"### {os.path.relpath(path)}: {steps} optimizer steps, {tot / max(steps, 1) / 1e6:.3f} ms of "
                  "kernel time per step\n")
            print("| kernel | calls | avg us | per step ms | share |\n|---|---|---|---|---|")
            for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
                t = float(r["TotalDurationNs"])
                name = _short_kernel_name(r["Name"])
                avg_us[name] = float(r["AverageNs"]) / 1e3
                print(f"| `{name}` | {r['Calls']} | {avg_us[name]:.1f} | "
                      f"{t / max(steps, 1) / 1e6:.3f} | {100 * t / tot:.2f}% |")
            print()
        for path in _find(folder, "counter_collection.csv"):
            per = {}  # (dispatch, kernel) -> {counter: value}
            for r in csv.DictReader(open(path)):
                d = per.setdefault((int(r["Dispatch_Id"]), r["Kernel_Name"]), {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            # the traffic probe's first three device copies move 1 GiB each
            copies = [d for (i, k), d in sorted(per.items()) if "copyBuffer" in k][:3]
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                vals = [d[c] for d in copies if c in d]
                if len(vals) == 3:
                    scale[c] = (1 << 20) / float(np.mean(vals))
            for (i, k), d in per.items():
                a = counters.setdefault(_short_kernel_name(k), {})
                for c, v in d.items():
                    s, n = a.get(c, (0.0, 0))
                    a[c] = (s + v, n + 1)
    if not counters:
        return
    mean = {k: {c: s / n for c, (s, n) in a.items()} for k, a in counters.items()}
    names = sorted(k for k in mean if "copyBuffer" not in k and "at::native" not in k)
    if scale:
        print("### HBM traffic per dispatch" + "".join(f"; {c} x {s:.3f}" for c, s in scale.items())
              + " (1 GiB copy)\n")
        print("| kernel | fetched MB | written MB | total MB | avg us | GB/s | of 8 TB/s |\n|---|---|---|---|---|---|---|")
        for k in names:
            m = mean[k]
            if "FETCH_SIZE" not in m and "WRITE_SIZE" not in m:
                continue
            f = m.get("FETCH_SIZE", 0.0) * scale.get("FETCH_SIZE", 1.0) * 1024 / 1e6
            w = m.get("WRITE_SIZE", 0.0) * scale.get("WRITE_SIZE", 1.0) * 1024 / 1e6
            us = avg_us.get(k)
            rate = (f + w) / us * 1e3 if us else None  # MB per us is TB/s
            print(f"| `{k}` | {f:,.1f} | {w:,.1f} | {f + w:,.1f} | " + (f"{us:.1f} | {rate:,.0f} | {rate / PEAK_HBM_GBS:.3f} |"
                                                                        if us else "- | - | - |"))
        print()
    if any("TCC_REQ_sum" in mean[k] for k in names):
        print("### L2 (TCC) requests per dispatch\n")
        print("| kernel | requests | hit rate | avg us | requests per us per XCD | x 128 B (TB/s) |\n|---|---|---|---|---|---|")
        for k in names:
            m = mean[k]
            if "TCC_REQ_sum" not in m:
                continue
            h, ms, q = m.get("TCC_HIT_sum", 0.0), m.get("TCC_MISS_sum", 0.0), m["TCC_REQ_sum"]
            us = avg_us.get(k)
            rate = f"{q / us / 8:,.0f} | {q * 128 / us / 1e6:.1f}" if us else "- | -"
            print(f"| `{k}` | {q:,.0f} | {h / (h + ms) if h + ms else 0.0:.3f} | " + (f"{us:.1f}" if us else "-")
                  + f" | {rate} |")
        print()
    busy_cols = [c for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT")
                 if any(c in mean[k] for k in names)]
    if busy_cols:
        print("### Issue counters per dispatch\n")
        raw = sorted({c for k in names for c in mean[k] if c not in ("FETCH_SIZE", "WRITE_SIZE") and not c.startswith("TCC_")})
        head = ["kernel"] + raw + ["MFMA busy", "dependency wait", "LDS conflict"]
        print("| " + " | ".join(head) + " |\n|" + "---|" * len(head))
        for k in names:
            m = mean[k]
            if not any(c in m for c in raw if c != "GRBM_GUI_ACTIVE"):
                continue
            cells = [f"`{k}`"] + [f"{m[c]:,.0f}" if c in m else "-" for c in raw]
            g_act = m.get("GRBM_GUI_ACTIVE", 0.0)
            mb = m.get("SQ_VALU_MFMA_BUSY_CYCLES")
            cells.append(f"{mb / (g_act / 8 * 1024):.3f}" if mb is not None and g_act else "-")
            cells.append(f"{m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.3f}"
                         if m.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in m else "-")
            cells.append(f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.3f}"
                         if m.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in m else "-")
            print("| " + " | ".join(cells) + " |")
        print()


def launch_work(cfg, B, T, esz, grouped, sr, n_unique):
    """Per timing point: the algorithmic work (FLOP or bytes) of each launch of
    one micro-step (forward + backward), or of one update for ADAMW."""
    L, C, Vp, P = cfg.num_layers, cfg.channels, cfg.padded_vocab_size, None
    BT = B * T
    att = 2.0 * B * T * (T + 1) * C  # causal: sum_t (t + 1) keys, two products
    w = {
        "CLASSIFIER_FWD": [2.0 * BT * Vp * C],
        "CLASSIFIER_DX": [2.0 * BT * Vp * C],
        "LAYER_FWD": [f for _ in range(L) for f in (2.0 * BT * C * 3 * C, 2.0 * BT * C * C,
                                                    2.0 * BT * C * 4 * C, 2.0 * BT * 4 * C * C)],
        "LAYER_DX": [f for _ in range(L) for f in (2.0 * BT * C * 4 * C, 2.0 * BT * 4 * C * C,
                                                   2.0 * BT * C * C, 2.0 * BT * 3 * C * C)],
        "ATTN_FWD": [att] * L,
        "ATTN_BWD": [2.0 * att] * L,  # dP, dV, dQ, dK (the recomputed scores not counted)
        # x read and y written, statistics written
        "LN_FWD": [2.0 * BT * C * esz + 8.0 * BT] * (2 * L + 1),
        # dy, x read; fp32 residual gradient read (not by the first) and
        # written; its low-precision copy written (bf16; not after layer 0)
        "LN_BWD": ([BT * C * (2 * esz + 4 + (esz if esz == 2 else 0)) + 8.0 * BT]
                   + [f for l in range(L - 1, -1, -1)
                      for f in (BT * C * (2 * esz + 8 + (esz if esz == 2 else 0)) + 8.0 * BT,
                                BT * C * (2 * esz + 8 + (esz if esz == 2 and l > 0 else 0)) + 8.0 * BT)]
                   # then the parameter gradients of all 2L + 1: their partial
                   # column sums (one row of 2C per workgroup of 16 rows, 32
                   # for rows of more than 96 16-byte vectors) read, dw and db
                   # read and written
                   + [(2 * L + 1) * (math.ceil(BT / (16 if math.ceil(C * esz / 16 / 32) <= 3 else 32)) * 2 * C * 4
                                     + 2 * 2 * C * 4)]),
        "CE": [2.0 * BT * Vp * esz + 8.0 * BT],
        # residual-gradient rows read, each present token's row read and
        # written, position rows read and written (fp32)
        "ENCODER_BWD": [4.0 * BT * C + 8.0 * n_unique * C + 8.0 * T * C],
    }
    if grouped:
        w["WEIGHT_GRAD"] = [2.0 * BT * C * (Vp + 12 * L * C)]
    else:
        w["WEIGHT_GRAD"] = [2.0 * BT * Vp * C] + w["LAYER_DX"]
    return w


def family_report(cfg, B, T, esz, grouped, sr, n_unique, P, times, n_micro, n_updates, step_ms):
    """times[point]: durations (ms) of every bracketed launch, in order."""
    per_call = launch_work(cfg, B, T, esz, grouped, sr, n_unique)
    per_call["ADAMW"] = [float(P) * (24 if sr else (30 if esz == 2 else 28))]
    out = []
    for name, point, bound in FAMILIES:
        t = times.get(point)
        if not t:
            continue
        wl = per_call[point]
        calls = n_updates if point == "ADAMW" else n_micro
        work = sum(wl) * calls
        ms = float(np.sum(t))
        if len(t) != len(wl) * calls:
            raise RuntimeError(f"{point}: {len(t)} bracketed launches, expected {len(wl) * calls}")
        steps = n_updates
        rate = work / (ms / 1e3)
        if bound == "mfma":
            peak = PEAK_BF16_TFLOPS if esz == 2 else PEAK_FP32_TFLOPS
            ach, unit = rate / 1e12, "TFLOP/s"
        else:
            peak = PEAK_HBM_GBS
            ach, unit = rate / 1e9, "GB/s"
        out.append({"family": name, "bound": bound, "launches_per_step": len(t) // steps,
                    "ms_per_step": round(ms / steps, 4), "share": round(ms / steps / step_ms, 4),
                    "achieved": round(ach, 1), "unit": unit, "peak": peak, "frac": round(ach / peak, 4)})
    return out


TRAFFIC_FILE = os.path.join(HERE, "profiles", "gpt2_124m_bf16_step_traffic.md")


def recorded_traffic(kernel_key):
    """HBM bytes per launch of a kernel of the step (FETCH_SIZE + WRITE_SIZE
    counter runs recorded in profiles/), if they were taken on the current
    GEMM source; else None."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = dict(l.split(":", 1) for l in text.splitlines() if ":" in l and not l.startswith(("|", " ", "#")))
    if vals.get("gemm_source_sha256", "").strip() != gemm_source_hash():
        return None
    try:
        return float(vals[f"traffic_bytes_per_launch {kernel_key}"])
    except (KeyError, ValueError):
        return None


def bench_gpt2(args):
    import torch
    import synthetic as S
    from transformer_lm_step_amd import binding as Bnd
    from transformer_lm_step_amd.model import GPT2

    big = args.model == "1558m"
    cfg = S.GPT2_1558M if big else S.GPT2_124M
    name = "1558M" if big else "124M"
    B, T = args.batch, args.seq
    # the 1.5B workload: 10 steps, lr 3e-4, no weight decay, no accumulation
    accum = 1 if big else args.accum
    lr, wd = (3e-4, 0.0) if big else (6e-4, 0.1)
    steps = args.steps if args.steps is not None else (10 if big else 20)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: GPT-2 {name} bf16 B={B} T={T} accum={accum} steps={steps} warmup={args.warmup}"
        + (" (no master weights, stochastic rounding)" if args.sr else ""))

    model = GPT2(cfg, Bnd.GPT2_BF16_SR if args.sr else Bnd.GPT2_BF16, B, T)
    params = {k: S.round_to_bf16(v) for k, v in S.init_params(cfg).items()}  # bf16-exact start
    model.init(model.pack(params))
    del params
    n_instr = 2  # instrumented steps after the timed ones
    n_micro = (args.warmup + steps + n_instr) * accum
    stream = S.token_stream(n_micro * B * T + 1, cfg.vocab_size, dist="zipf")
    toks = torch.from_numpy(stream).to(dev)
    BT = B * T
    xs = [toks[i * BT:(i + 1) * BT] for i in range(n_micro)]
    ys = [toks[i * BT + 1:(i + 1) * BT + 1].clone() for i in range(n_micro)]
    mean_loss = torch.zeros(n_micro, dtype=torch.float32, device=dev)
    dloss = 1.0 / (accum * BT)

    def step(s):
        model.zero_grad()
        for a in range(accum):
            i = s * accum + a
            model.forward(xs[i], ys[i], None, mean_loss[i:i + 1])
            model.backward(dloss)
        model.update(lr, 0.9, 0.999, 1e-8, wd, s + 1)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    if model.check() != 0:
        raise RuntimeError("device-side error during warmup")
    log("bench: warmup done")

    # HIP events around the weight-gradient launch of every backward in the
    # timed steps (recorded by the library on the step's stream)
    hip = HipEvents()
    n_ev = steps * accum
    starts, ends = hip.create(n_ev), hip.create(n_ev)
    hook = Bnd.gpt2_set_timing_events(model.ctx, Bnd.GPT2_TP_WEIGHT_GRAD, starts, ends)
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # one event between consecutive steps: per-step times for the median
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps - 1)]
    e0.record(cur)
    for i, s in enumerate(range(args.warmup, args.warmup + steps)):
        step(s)
        if i < steps - 1:
            marks[i].record(cur)
    e1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    Bnd.gpt2_set_timing_events(model.ctx, Bnd.GPT2_TP_WEIGHT_GRAD, [], [])
    del hook
    ms = e0.elapsed_time(e1) / steps
    bounds = [e0] + marks + [e1]
    step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps)]
    ms_median = float(np.median(step_ms))
    losses = mean_loss[:(args.warmup + steps) * accum].cpu().numpy()
    if not np.all(np.isfinite(losses)):
        raise RuntimeError("non-finite loss")
    tok_s = accum * BT / (ms / 1e3)
    fpt = flops_per_token(cfg.num_layers, cfg.channels, cfg.vocab_size, T)
    mfu = tok_s * fpt / (PEAK_BF16_TFLOPS * 1e12)
    # the common 6N + 12 L C T convention (N = every parameter, embeddings included)
    fpt_6n = 6.0 * model.num_params + 12.0 * cfg.num_layers * cfg.channels * T
    mfu_6n = tok_s * fpt_6n / (PEAK_BF16_TFLOPS * 1e12)
    log(f"bench: {ms:.3f} ms/step (median {ms_median:.3f}), {tok_s:,.0f} tok/s, MFU {mfu:.3f} "
        f"(6N+12LCT: {mfu_6n:.3f}), wall {wall:.2f}s, "
        f"loss first {losses[0]:.4f} last {losses[-1]:.4f}")

    # ---- dominant kernel: the weight-gradient launches of a micro-step (one
    # grouped launch, followed by the attention projections' own launch on
    # 128x256 tiles where that saves a round of tiles), inside the timed steps
    kms = float(np.mean([hip.elapsed_ms(a, b) for a, b in zip(starts, ends)]))
    hip.destroy(starts + ends)
    L, C, Vp = cfg.num_layers, cfg.channels, cfg.padded_vocab_size
    kflop = 2.0 * BT * C * (Vp + 12 * L * C)
    achieved = kflop / (kms / 1e3) / 1e12
    traffic = recorded_traffic("weight_grad") if (not big and (B, T) == (8, 1024)) else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": f"gemm_dtl_kernel, grouped weight gradients (classifier {Vp}x{C} + {L} layers x "
                          f"4 products, K = B*T = {BT}, bf16, in-step launches; the attention projections "
                          f"in a second launch on 128x256 tiles where that saves a round)",
                "avg_ms": round(kms, 4), "launches": n_ev}
    log(f"bench: weight-gradient launch in the step {kms:.3f} ms, {achieved:.1f} TFLOP/s")

    # ---- every kernel family, from n_instr further steps with all hooks set
    points = {p: getattr(Bnd, "GPT2_TP_" + p) for _, p, _ in FAMILIES}
    n_unique = int(np.mean([np.unique(stream[i * BT:(i + 1) * BT]).size for i in range(n_micro)]))
    work = launch_work(cfg, B, T, 2, True, args.sr, n_unique)
    evs = {}
    for _, p, _ in FAMILIES:
        per = 1 if p == "ADAMW" else len(work[p]) * accum
        n = per * n_instr
        evs[p] = (hip.create(n), hip.create(n))
    hooks = [Bnd.gpt2_set_timing_events(model.ctx, points[p], a, b) for p, (a, b) in evs.items()]
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(cur)
    for s in range(args.warmup + steps, args.warmup + steps + n_instr):
        step(s)
    e3.record(cur)
    torch.cuda.synchronize()
    for p in points:
        Bnd.gpt2_set_timing_events(model.ctx, points[p], [], [])
    del hooks
    instr_ms = e2.elapsed_time(e3) / n_instr
    times = {p: [hip.elapsed_ms(a, b) for a, b in zip(sa, ea)] for p, (sa, ea) in evs.items()}
    for sa, ea in evs.values():
        hip.destroy(sa + ea)
    families = family_report(cfg, B, T, 2, True, args.sr, n_unique, model.num_params, times,
                             n_instr * accum, n_instr, instr_ms)
    for f in families:
        log(f"bench:   {f['family']:55s} {f['ms_per_step']:8.3f} ms/step  {f['achieved']:8.1f} {f['unit']:8s} "
            f"frac {f['frac']:.3f}")
    peak_hbm = torch.cuda.max_memory_allocated(dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle sample ...")
        cpu = cpu_baseline(cfg, 256, name) if not big else cpu_baseline(cfg, 16, name)
        log(f"bench: oracle {cpu['value']:.3f} tok/s ({cpu['sample']}; host {cpu['host_cpu']}, "
            f"{cpu['host_nproc']} logical cores)")

    workload = (f"GPT-2 {name} training step: {accum} micro-step{'s' if accum > 1 else ''} of B={B} T={T} + "
                f"AdamW (lr {lr:g}, wd {wd:g})")
    out = {
        "metric": f"train tokens/sec + MFU, GPT-2 {name} bf16 B={B} T={T} on 1x MI355X"
                  + (" (bf16 parameters without master weights, stochastic rounding)" if args.sr else ""),
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (Zipf(1.1) token stream, random GPT-2 init)",
        "config": {"workload": workload, "global_batch": accum * B, "seq_len": T, "grad_accum": accum,
                   "parallelism": "single GPU"},
        "ms_per_step_median": round(ms_median, 4),
        "mfu": round(mfu, 4),
        "flops_per_token": fpt,
        "mfu_6n": round(mfu_6n, 4),
        "flops_per_token_6n": fpt_6n,
        "roofline": roofline,
        "families": families,
        "instrumented_ms_per_step": round(instr_ms, 4),
        "peak_hbm_gb": round(peak_hbm / 1e9, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    model.close()


def bench_c2(args):
    """GPT-2 124M in fp32 (full fp32 products), B=4 T=64, 10 AdamW steps (lr
    1e-4, wd 0) overfitting one batch: tokens/s and the fraction of the fp32
    peak the step's algorithmic FLOPs reach; the oracle times one of the same
    steps on the host."""
    import torch
    import synthetic as S
    from transformer_lm_step_amd import binding as Bnd
    from transformer_lm_step_amd.model import GPT2

    cfg, B, T = S.GPT2_124M, 4, 64
    steps = args.steps if args.steps is not None else 10
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = GPT2(cfg, Bnd.GPT2_FP32, B, T)
    model.init(model.pack(S.init_params(cfg)))
    stream = S.token_stream(B * T + 1, cfg.vocab_size, dist="zipf")
    xb, yb = S.batch(stream, 0, B, T)
    x = torch.from_numpy(xb.reshape(-1)).to(dev)
    y = torch.from_numpy(yb.reshape(-1)).to(dev)
    mean = torch.zeros(args.warmup + steps, dtype=torch.float32, device=dev)

    def step(s):
        model.zero_grad()
        model.forward(x, y, None, mean[s:s + 1])
        model.backward(1.0 / (B * T))
        model.update(1e-4, 0.9, 0.999, 1e-8, 0.0, s + 1)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for s in range(args.warmup, args.warmup + steps):
        step(s)
    e1.record(cur)
    torch.cuda.synchronize()
    if model.check() != 0:
        raise RuntimeError("device-side error")
    ms = e0.elapsed_time(e1) / steps
    lo = mean.cpu().numpy()
    tok_s = B * T / (ms / 1e3)
    fpt = flops_per_token(cfg.num_layers, cfg.channels, cfg.vocab_size, T)
    frac = tok_s * fpt / (PEAK_FP32_TFLOPS * 1e12)
    log(f"bench: c2 fp32 {ms:.3f} ms/step, {tok_s:,.0f} tok/s, {frac:.4f} of the fp32 peak, "
        f"loss {lo[0]:.4f} -> {lo[-1]:.4f}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        flat = oracle.pack_params(cfg, S.init_params(cfg))
        t0 = time.perf_counter()
        oracle.gpt2_step(cfg, flat, xb, yb, dloss=1.0 / (B * T))
        dt = time.perf_counter() - t0
        model_name, ncpu = host_cpu()
        cpu = {"value": round(B * T / dt, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"one of the same steps (forward + backward, B=4 T=64, fp64, single thread), {dt:.1f} s",
               "host_cpu": model_name, "host_nproc": ncpu}
    out = {
        "metric": "train tokens/sec, GPT-2 124M fp32 B=4 T=64 (10 steps on one batch) on 1x MI355X",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (Zipf(1.1) tokens, random GPT-2 init)",
        "config": {"workload": "GPT-2 124M fp32 training step, B=4 T=64, AdamW lr 1e-4 wd 0, one batch"},
        "fp32_peak_frac": round(frac, 5), "flops_per_token": fpt,
        "roofline": {"bound": "mfma", "achieved": round(tok_s * fpt / 1e12, 2), "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(frac, 5), "traffic": None,
                     "kernel": "whole step (algorithmic FLOPs / step time)", "avg_ms": round(ms, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    model.close()


if __name__ == "__main__":
    main()
