#!/usr/bin/env python
"""Decode benchmark of the windowed INT8 recurrent-state path on one MI355X.

One step = one decode token for every (sequence, head) unit of every layer
(lq_decode_step), plus the window-boundary requantization (lq_window_flush)
for every unit whose window filled on that token.  Inputs are synthetic,
seeded, and resident in HBM before the timed region starts.  The timed steps
are captured as one HIP graph and replayed between HIP events (median of
--repeats replays), so the host's launch cost is not in the figure.  The same
steps are then timed on the FP32-state comparison kernel.  --replicas R runs
every step on R independent copies of the states in turn, which pushes a
working set that would fit the 256 MB last-level cache out to HBM.

Prints one JSON line:
  value            unit-tokens/s (seq·head·tokens/s) of the INT8 path over the timed steps
  roofline         the decode kernel's algorithmic bytes per launch / its average
                   launch time (a graph of one window of decode launches, HIP events
                   around the replay), against 8 TB/s; `practical` adds what a plain
                   streaming-read kernel reaches on this device at the same bytes
                   per launch (probe/stream_read, run after the timed region)
  fp32_state       the FP32-state kernel on the same steps, and the speedup
  cpu_baseline     the CPU oracle (FP64, definitional windowed form) on a bounded
                   sample of the same workload, on this host's cores
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "seq·head·tokens/s decode; HBM GB/s vs peak; speedup vs FP32-state kernel"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode tokens (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed tokens first (default: one window)")
    ap.add_argument("--workload", default="gdn_decode",
                    help="tiny_gdn | gdn_decode | kda_decode | gdn_serving | hybrid_stack")
    ap.add_argument("--window", type=int, default=None, help="override the workload's window W (1..256)")
    ap.add_argument("--n-comp", type=int, default=None, help="override the workload's compensator count (0..16)")
    ap.add_argument("--format", default="int8", choices=("int8", "e4m3"),
                    help="8-bit code format of the stored state")
    ap.add_argument("--buffer", default="fp32", choices=("fp32", "fp16"),
                    help="precision of the window buffer's k and v")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-fp32", action="store_true", help="skip the FP32-state comparison loop")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip timing lq_prefill on the workload's prompt against the token-by-token FP32 kernel")
    ap.add_argument("--repeats", type=int, default=5,
                    help="replays of the timed-steps graph, median reported (1 if the steps are not whole "
                         "windows: only then does a replay restart the same fill pattern)")
    ap.add_argument("--replicas", type=int, default=1,
                    help="independent copies of every state, each token run on every copy in turn: with "
                         "enough copies the working set exceeds the 256 MB last-level cache, so every launch "
                         "reads its state from HBM (throughput counts the units of all copies)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic byte model (what the method must move, per unit and token)
# ---------------------------------------------------------------------------

def entry_bytes(wl) -> int:
    g = wl.d if wl.gate == "channel" else 1
    e = 2 if wl.buffer_format == "fp16" else 4  # k and v elements
    return e * (wl.d // wl.group + wl.d) + 4 * (1 + g)


def decode_bytes(wl, j: int) -> int:
    """Bytes one unit moves in one decode step with j tokens already buffered."""
    d, nc = wl.d, wl.n_comp
    g = d if wl.gate == "channel" else 1
    E = entry_bytes(wl)
    tile = d * d + 4 * (2 * d) + nc * (4 * d + 4)
    inputs = 4 * (2 * d // wl.group + d + 1 + g)
    return tile + j * E + inputs + E + 4 * d + 8


def flush_bytes(wl, n: int) -> int:
    """Bytes one unit moves in one flush over n buffered tokens (read and rewrite the stored state)."""
    d, nc = wl.d, wl.n_comp
    stored = d * d + 4 * 2 * d + nc * (4 * d + 4)
    return 2 * stored + n * entry_bytes(wl) + 8


# ---------------------------------------------------------------------------
# inputs on the device
# ---------------------------------------------------------------------------

def device_tokens(wl, n_tok, layer, gen, dev, weights=None):
    import torch

    from linear_attention_recurrent_gdn_amd import inputs as I

    out = []
    for _ in range(n_tok):
        if wl.projected:
            h = torch.randn((wl.n_seq, wl.hidden), generator=gen, device=dev).to(torch.bfloat16)
            out.append(projected(wl, weights, h))
        else:
            out.append(I.torch_token(wl, gen, dev))
    return out


def projection_weights(wl, gen, dev):
    import torch

    std = 1.0 / wl.hidden ** 0.5
    KH, H, d = wl.n_k_heads, wl.n_v_heads, wl.d
    return {name: (torch.randn((n, wl.hidden), generator=gen, device=dev) * std).to(torch.bfloat16)
            for name, n in (("wq", KH * d), ("wk", KH * d), ("wv", H * d), ("wa", H), ("wb", H))}


def projected(wl, w, h):
    """q, k, v, beta, alpha from a bf16 hidden state (input synthesis, not the timed path)."""
    import torch

    S, KH, H, d = wl.n_seq, wl.n_k_heads, wl.n_v_heads, wl.d
    p = lambda name: (h @ w[name].t().contiguous()).float()
    q = p("wq").view(S, KH, d)
    k = p("wk").view(S, KH, d)
    return {"q": (q / q.norm(dim=-1, keepdim=True)).contiguous(),
            "k": (k / k.norm(dim=-1, keepdim=True)).contiguous(),
            "v": p("wv").view(S, H, d).contiguous(),
            "beta": torch.sigmoid(p("wb")).contiguous(),
            "gate": (0.9 + 0.1 * torch.sigmoid(p("wa"))).contiguous()}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(wl, n_tok, target_s, fmt="int8", buffer="fp32"):
    import numpy as np

    import oracle as orc
    from linear_attention_recurrent_gdn_amd import inputs as I

    src = wl.scaled(projected=False) if wl.projected else wl

    def sample(units, n):
        st = I.prefill_streams(src, units, n=n, phase=I.PHASE_DECODE, with_queries=True)
        S0 = I.surrogate_state(src, units).astype(np.float64)
        return S0, st

    # calibrate on a few units, then size the sample for about target_s seconds
    cal_units = list(range(min(2 * orc.num_threads(), wl.n_units)))
    cal_tok = min(n_tok, 2 * wl.window)
    S0, st = sample(cal_units, cal_tok)
    t0 = time.perf_counter()
    orc.windowed_run(S0, st["q"], st["k"], st["v"], st["beta"], st["gate"], wl.window, wl.n_comp, fmt=fmt,
                     buffer=buffer)
    rate = len(cal_units) * cal_tok / max(time.perf_counter() - t0, 1e-6)
    n_units = int(max(1, min(wl.n_units, rate * target_s / n_tok)))
    # the whole workload may take well under target_s: repeat it to get a steady figure
    reps = int(max(1, min(20, round(rate * target_s / (n_units * n_tok)))))
    units = np.linspace(0, wl.n_units - 1, n_units).astype(int)
    S0, st = sample(units, n_tok)
    t0 = time.perf_counter()
    for _ in range(reps):
        orc.windowed_run(S0, st["q"], st["k"], st["v"], st["beta"], st["gate"], wl.window, wl.n_comp, fmt=fmt,
                         buffer=buffer)
    dt = time.perf_counter() - t0
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except Exception:
        pass
    return {
        "value": reps * n_units * n_tok / dt,
        "unit": "seq·head·tokens/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": (f"{n_units} of {wl.n_units} units x {n_tok} decode tokens (flushes included) x {reps} passes, "
                   f"FP64 definitional windowed form, {dt:.1f} s; input generation excluded; "
                   f"host CPU: {cpu_model}"),
    }


# ---------------------------------------------------------------------------
# prefill: the chunked FP64 matrix-core prompt pass against the FP32 token loop
# ---------------------------------------------------------------------------

PEAK_FP64_MFMA_TFLOPS = 78.6


def prefill_flops(wl, n_tok) -> float:
    """Matrix-core flops of the chunked prompt pass per unit: per token the
    products T Kf^T, T Qf^T and the rank-16 update C Kb (2 d^2 each), per
    16-token chunk the two 16 x 16 x d Gram products, M R and the output
    correction (2 * 16 * 16 * d each)."""
    d = wl.d
    chunks = -(-n_tok // 16)
    return n_tok * 6.0 * d * d + chunks * 4 * (2.0 * 16 * 16 * d)


def prefill_timing(lq, wl, cfg, gen, dev, timed_graph):
    import torch

    from linear_attention_recurrent_gdn_amd import inputs as I

    P, U, d = wl.prefill, wl.n_units, wl.d
    first = I.torch_token(wl, gen, dev)
    x = {k: torch.empty((P, *v.shape), dtype=v.dtype, device=dev) for k, v in first.items()}
    for t in range(P):
        tk = first if t == 0 else I.torch_token(wl, gen, dev)
        for k in x:
            x[k][t].copy_(tk[k])
    S0 = torch.randn((U, d, d), generator=gen, device=dev) * 0.3
    o = torch.empty((P, wl.n_seq, wl.n_v_heads, d), device=dev)
    blob = lq.new_state(cfg, dev)
    chunked_ms = timed_graph(lambda: lq.lq_prefill(cfg, blob, S0, x["q"], x["k"], x["v"], x["beta"], x["gate"], o),
                             3)
    S = S0.clone()
    o1 = torch.empty((wl.n_seq, wl.n_v_heads, d), device=dev)
    loop_ms = timed_graph(lambda: [lq.lq_fp32_decode_step(cfg, S, x["q"][t], x["k"][t], x["v"][t], x["beta"][t],
                                                          x["gate"][t], o1) for t in range(P)])
    if lq.lq_read_status(cfg, blob):
        raise RuntimeError("device flags set by lq_prefill")
    flops = prefill_flops(wl, P) * U
    return {
        "tokens": P, "units": U,
        "chunked_ms": chunked_ms,
        "fp32_token_loop_ms": loop_ms,
        "speedup": loop_ms / chunked_ms,
        "unit_tokens_per_s": P * U / (chunked_ms * 1e-3),
        "roofline": {"bound": "mfma", "achieved": flops / (chunked_ms * 1e-3) / 1e12,
                     "peak": PEAK_FP64_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / (chunked_ms * 1e-3) / 1e12 / PEAK_FP64_MFMA_TFLOPS,
                     "kernel": "materialize_kernel (prefill mode)", "dtype": "f64"},
        "note": "lq_prefill (outputs written, final state quantized) vs the FP32 decode kernel token by token "
                "over the same prompt from the same start state; each as one HIP graph",
    }


# ---------------------------------------------------------------------------
# measured HBM traffic (rocprofv3 --pmc), valid only for the kernel it was taken on
# ---------------------------------------------------------------------------

def practical_read(nbytes: float):
    """Best rate of the plain streaming-read probe (16-byte loads, grid-stride,
    nothing else) over its grid sizes at `nbytes` per launch, in GB/s, or None
    when the probe is not built.  Runs as a child process after the timed work."""
    import subprocess

    from linear_attention_recurrent_gdn_amd import _build

    if not os.path.exists(_build.PROBE):
        return None
    r = subprocess.run([_build.PROBE, str(int(nbytes))], capture_output=True, text=True, timeout=120)
    rows = [json.loads(line) for line in r.stdout.splitlines() if line.startswith("{")]
    if r.returncode != 0 or not rows:
        return None
    best = max(rows, key=lambda x: x["TBps"])
    return {"GBps": best["TBps"] * 1e3, "us": best["us"], "grid": best["grid"]}


def variant_tag(workload, fmt="int8", buffer="fp32"):
    """Name of a workload variant in profile file names."""
    return workload + ("" if fmt == "int8" else f"_{fmt}") + ("" if buffer == "fp32" else f"_{buffer}buf")


def measured_traffic(workload, fmt="int8", buffer="fp32"):
    p = os.path.join(ROOT, "profiles", f"decode_q8_{variant_tag(workload, fmt, buffer)}_traffic.json")
    try:
        rec = json.load(open(p))
    except Exception:
        return None
    from linear_attention_recurrent_gdn_amd.profiling import kernel_sha

    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------

def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); units shard across GPUs with no exchange, "
              f"so the per-GPU figure is the N=1 line.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import linear_attention_recurrent_gdn_amd as lq
    from linear_attention_recurrent_gdn_amd import inputs as I

    lq.load_library()
    wl = I.WORKLOADS[args.workload]
    if args.window is not None:
        wl = wl.scaled(window=args.window)
    if args.n_comp is not None:
        wl = wl.scaled(n_comp=args.n_comp)
    wl = wl.scaled(code_format=args.format, buffer_format=args.buffer)
    W, U, L, d = wl.window, wl.n_units, wl.layers, wl.d
    steps = wl.decode if args.steps is None else args.steps
    warmup = W if args.warmup is None else args.warmup
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(dev).manual_seed(1000 + wl.seed)
    code_format = {"int8": lq.LQ_CODE_INT8, "e4m3": lq.LQ_CODE_E4M3}[args.format]
    buffer_format = {"fp32": lq.LQ_BUFFER_FP32, "fp16": lq.LQ_BUFFER_FP16}[args.buffer]
    cfg = lq.Config(wl.n_seq, wl.n_v_heads, wl.n_k_heads, d, d, W, wl.n_comp, wl.gate_kind, code_format,
                    buffer_format)
    stream = torch.cuda.current_stream()

    # ---- start states: FP32 prefill through the FP32-state kernel (input synthesis)
    weights = [projection_weights(wl, gen, dev) for _ in range(L)] if wl.projected else [None] * L
    S_fp32, states = [], []
    o = torch.empty((wl.n_seq, wl.n_v_heads, d), device=dev)
    for layer in range(L):
        S = torch.zeros((U, d, d), device=dev)
        for tk in device_tokens(wl, wl.prefill, layer, gen, dev, weights[layer]):
            lq.lq_fp32_decode_step(cfg, S, tk["q"], tk["k"], tk["v"], tk["beta"], tk["gate"], o)
        sc = I.outlier_scale(wl, layer)
        if sc is not None:
            r, c = (torch.from_numpy(x).to(dev) for x in sc)
            S *= r[:, :, None] * c[:, None, :]
        st = lq.new_state(cfg, dev)
        lq.lq_state_init(cfg, st, S)
        states.append(st)
        S_fp32.append(S)
    R = max(1, args.replicas)
    blobs = [[st] + [st.clone() for _ in range(R - 1)] for st in states]  # [layer][copy]
    if not args.no_fp32:
        S_fp32 = [[S] + [S.clone() for _ in range(R - 1)] for S in S_fp32]
    n_tok = warmup + steps
    toks = [device_tokens(wl, n_tok, layer, gen, dev, weights[layer]) for layer in range(L)]
    torch.cuda.synchronize()

    sched = I.stagger_schedule(wl)
    fill = np.zeros(wl.n_seq, np.int64)
    force_dev = torch.zeros(wl.n_seq, dtype=torch.uint8, device=dev)
    flush_calls = []

    def q8_step(t):
        for layer in range(L):
            tk = toks[layer][t]
            for st in blobs[layer]:
                lq.lq_decode_step(cfg, st, tk["q"], tk["k"], tk["v"], tk["beta"], tk["gate"], o)
        fill[:] += 1
        forced = (sched == t) if (sched is not None and t < warmup) else np.zeros(wl.n_seq, bool)
        due = (fill >= W) | (forced & (fill > 0))
        if due.any():
            fm = None
            if forced.any():
                force_dev.copy_(torch.from_numpy(forced.astype(np.uint8)))
                fm = force_dev
            for layer in range(L):
                for st in blobs[layer]:
                    lq.lq_window_flush(cfg, st, fm)
            flush_calls.append(int(due.sum()) * wl.n_v_heads)
            fill[due] = 0

    def timed_graph(body, repeats=1):
        """Capture body() as one HIP graph, replay it `repeats` times, each between
        HIP events; the median replay time (ms)."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        torch.cuda.synchronize()
        times = []
        for _ in range(max(1, repeats)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        del g
        return float(np.median(times))

    for t in range(warmup):
        q8_step(t)
    n_flush_warm = len(flush_calls)
    # the timed steps run as one graph: kernels back to back, no host launch cost
    repeats = args.repeats if steps % W == 0 else 1
    q8_ms = timed_graph(lambda: [q8_step(t) for t in range(warmup, n_tok)], repeats)
    flags = [lq.lq_read_status(cfg, st) for bl in blobs for st in bl]
    if any(flags):
        raise RuntimeError(f"device flags set during the run: {flags}")

    result = {
        "metric": METRIC,
        "value": U * L * R * steps / (q8_ms * 1e-3),
        "unit": "seq·head·tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": q8_ms / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "state_dtype": args.format,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "layers": L, "n_seq": wl.n_seq, "n_v_heads": wl.n_v_heads, "n_k_heads": wl.n_k_heads,
            "d_k": d, "d_v": d, "gate": wl.gate, "window": W, "n_comp": wl.n_comp,
            "code_format": args.format, "buffer_format": args.buffer,
            "prefill": wl.prefill, "units": U * L * R, "state_copies": R,
        },
        "timing": f"HIP graph of the timed steps, median of {repeats} replays, HIP events around each",
    }

    # ---- the decode kernel alone over one whole window (every unit at j = 0 .. W-1),
    # replayed as a graph: its average launch time against its algorithmic bytes
    all_seq = torch.ones(wl.n_seq, dtype=torch.uint8, device=dev)
    for bl in blobs:
        for st in bl:
            lq.lq_window_flush(cfg, st, all_seq)  # forced: every window restarts empty
    win_tok = [t % n_tok for t in range(W)]
    dec_ms = timed_graph(lambda: [lq.lq_decode_step(cfg, st, toks[layer][t]["q"], toks[layer][t]["k"],
                                                    toks[layer][t]["v"], toks[layer][t]["beta"],
                                                    toks[layer][t]["gate"], o)
                                  for t in win_tok for layer in range(L) for st in blobs[layer]])
    n_launch = W * L * R
    avg_launch_s = dec_ms * 1e-3 / n_launch
    avg_bytes = float(np.mean([decode_bytes(wl, j) for j in range(W)])) * U
    achieved = avg_bytes / avg_launch_s / 1e9
    result["roofline"] = {
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        "traffic": measured_traffic(wl.name, args.format, args.buffer),
        "kernel": "decode_q8_kernel",
        "avg_launch_us": avg_launch_s * 1e6,
        "alg_bytes_per_launch": avg_bytes,
        "launches": n_launch,
        "note": "one graph of one window of decode launches (j = 0..W-1), events around the replay",
    }
    # flush alone: one forced boundary of every unit after a full window
    fl_ms = timed_graph(lambda: [lq.lq_window_flush(cfg, blobs[layer][0], None) for layer in range(L)])
    result["flush"] = {
        "avg_launch_us": fl_ms * 1e3 / L,
        "units_per_launch": U,
        "tokens_replayed": W,
        "timed_steps_flushes": len(flush_calls) - n_flush_warm,
    }

    if not args.no_fp32:
        def fp32_steps(t_from, t_to):
            for t in range(t_from, t_to):
                for layer in range(L):
                    tk = toks[layer][t]
                    for S in S_fp32[layer]:
                        lq.lq_fp32_decode_step(cfg, S, tk["q"], tk["k"], tk["v"], tk["beta"], tk["gate"], o)
        fp32_steps(0, warmup)
        fp32_ms = timed_graph(lambda: fp32_steps(warmup, n_tok), repeats)
        fp32_bytes = U * L * R * (8 * d * d + 4 * (2 * d // wl.group + 2 * d + 1 + (d if wl.gate == "channel" else 1)))
        result["fp32_state"] = {
            "value": U * L * R * steps / (fp32_ms * 1e-3),
            "ms_per_step": fp32_ms / steps,
            "alg_GBps": fp32_bytes / (fp32_ms / steps * 1e-3) / 1e9,
            "speedup_vs_fp32": fp32_ms / q8_ms,
        }

    if not args.no_prefill and wl.prefill > 0 and not wl.projected and L == 1:
        result["prefill"] = prefill_timing(lq, wl, cfg, gen, dev, timed_graph)

    # the practical ceiling at the decode launch's byte count (a child process;
    # the device is idle here)
    torch.cuda.synchronize()
    pr = practical_read(avg_bytes)
    if pr is not None:
        result["roofline"]["practical"] = {
            "kernel": "stream_read (probe/stream_read.hip): 16-byte loads, grid-stride, nothing else",
            "bytes_per_launch": avg_bytes, "achieved": pr["GBps"], "unit": "GB/s",
            "frac_of_peak": pr["GBps"] / HBM_PEAK_GBS, "decode_frac_of_practical": achieved / pr["GBps"],
        }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, steps, args.cpu_seconds, args.format, args.buffer)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
