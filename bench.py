#!/usr/bin/env python
"""Decode benchmark of the windowed INT8 recurrent-state path on one MI355X.

One step = one decode token for every (sequence, head) unit of every layer
(lq_decode_step), plus the window-boundary requantization (lq_window_flush)
of every layer whose units filled their window on that token.  Inputs are
synthetic, seeded, and resident in HBM before the timed region starts.

Boundary beside the decode.  With several layers, a layer's boundary call
depends only on that layer's decode of the token, and only that layer's next
decode depends on it; it runs on a second stream (--flush-cus: its persistent
grid limited to 96 of the 256 CUs by default) while the next layers decode on
the rest, and the layer's next decode waits for it through an event.

Steady state.  Windows are staggered so that any run of steps carries its
share of boundary work and sees every fill position of the window: with
several layers, layer l starts its windows floor(l W / L) tokens later than
layer 0 (every layer flushes all its units once per W steps, at different
steps); with one layer, sequences are split into G groups at offsets g W / G
(G up to 8, each group at least 256 units, one per CU); a workload defined
with per-sequence offsets (the serving step) keeps them.  A set-up phase of
W untimed tokens (forced flushes) establishes the offsets, then --warmup
untimed steps run, then --steps steps are timed.  The timed steps run as HIP
graphs of --steps steps each, captured and replayed once per segment, for
--repeats consecutive segments (HIP events around each replay); the median
segment gives ms_per_step, so the host's launch cost is not in the figure.
The same steps then run on the FP32-state comparison kernel.  --replicas R
runs every step on R independent copies of the states in turn, which pushes
a working set that would fit the 256 MB last-level cache out to HBM.

Prints one JSON line:
  value            unit-tokens/s (seq.head.tokens/s, all layers) of the INT8 path,
                   window-boundary requantization included
  roofline         the decode kernel: algorithmic bytes per launch / its average
                   launch time (a graph of one window of decode launches, every
                   layer at fill 0 .. W-1, HIP events around the replay), against
                   8 TB/s; `practical` adds what a plain streaming-read kernel
                   reaches from HBM on this device at the same bytes per launch
  flush            the boundary kernel alone (all units of a layer after a full
                   window) and its FP64 matrix-core roofline (5 d^2 W flop per unit)
  checks           ms_per_step against the decode launches it must contain, and
                   the speedup against the byte-ratio ceiling
  fp32_state       the FP32-state kernel on the same steps, and the speedup
  cpu_baseline     the CPU oracle (FP64, definitional windowed form) on a bounded
                   sample of the same workload: all host threads, and one thread
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
METRIC = "seq·head·tokens/s decode; HBM GB/s vs peak; speedup vs FP32-state kernel"


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps per segment (default: the workload's "
                                                            "decode tokens)")
    ap.add_argument("--warmup", type=int, default=8, help="untimed steps after the set-up phase")
    ap.add_argument("--workload", default="hybrid_stack",
                    help="tiny_gdn | gdn_decode | kda_decode | gdn_serving | hybrid_stack")
    ap.add_argument("--window", type=int, default=None, help="override the workload's window W (1..256)")
    ap.add_argument("--n-comp", type=int, default=None, help="override the workload's compensator count (0..16)")
    ap.add_argument("--format", default="int8", choices=("int8", "e4m3"),
                    help="8-bit code format of the stored state")
    ap.add_argument("--buffer", default="fp32", choices=("fp32", "fp16", "nform"),
                    help="window buffer: k and v in fp32 or binary16, or the chain-free form (fp32 k and n; "
                         "scalar gate, d = 128)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-fp32", action="store_true", help="skip the FP32-state comparison loop")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip timing lq_prefill on the workload's prompt against the token-by-token FP32 kernel")
    ap.add_argument("--repeats", type=int, default=5,
                    help="consecutive timed segments of --steps steps, each one HIP graph replayed once; "
                         "the median is reported")
    ap.add_argument("--replicas", type=int, default=1,
                    help="independent copies of every state, each token run on every copy in turn: with "
                         "enough copies the working set exceeds the 256 MB last-level cache, so every launch "
                         "reads its state from HBM (throughput counts the units of all copies)")
    ap.add_argument("--flush-cus", type=int, default=-1,
                    help="multi-layer workloads: run each layer's boundary call on a second stream, on this many "
                         "CUs (lq_config.flush_cus), beside the next layers' decode steps; 0 runs it on the "
                         "decode stream after the token's last layer; -1 (default) picks 96 of 256, 128 with the binary16 "
                         "buffer (measured best of 64-160)")
    ap.add_argument("--load-policy", default="residency", choices=("residency", "auto", "stream", "cached"),
                    help="lq_config.load_policy of the decode steps: streaming (non-temporal) state reads, "
                         "automatic (launches of more than 2,048 units), or ordinary; 'residency' (default) "
                         "streams when the states of every layer and copy exceed twice the 256 MB "
                         "last-level cache, as a caller that knows its working set would, else automatic")
    ap.add_argument("--stagger-layout", default="blocks", choices=("blocks", "interleaved"),
                    help="one-layer workloads: which sequences share a window offset (consecutive ones, "
                         "fills falling along the unit index; or sequence s in group s mod G)")
    return ap.parse_args(argv)


# ---------------------------------------------------------------------------
# algorithmic byte model (what the method must move, per unit and token)
# ---------------------------------------------------------------------------

def entry_bytes(wl) -> int:
    g = wl.d if wl.gate == "channel" else 1
    if wl.buffer_format == "nform":  # k, the vector n and the gate (beta is inside n)
        return 4 * (wl.d // wl.group + wl.d) + 4 * g
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
# staggered windows: the host mirror of every (layer, sequence)'s fill count
# ---------------------------------------------------------------------------

def stagger_groups(wl) -> int:
    """Groups of sequences at distinct window offsets in a one-layer workload:
    the most (up to 8) that divide the window and the sequences and leave at
    least 256 units (one per CU) to each group's boundary launch."""
    for G in (8, 4, 2):
        if wl.window % G == 0 and wl.n_seq % G == 0 and wl.n_units // G >= 256:
            return G
    return 1


def window_offsets(wl, n_layers, layout="blocks"):
    """Fill count [layer, sequence] after the set-up phase (the window offsets).

    One layer: G groups of sequences at offsets W/G apart (G = W for a workload
    defined with per-sequence offsets, the serving step).  `layout` says which
    sequences share an offset: "blocks", consecutive sequences, with the
    offsets falling along the sequence index (so along the unit index, and
    the decode launch's dispatch order, fills fall too, with one wrap), or
    "interleaved", sequence s in group s mod G."""
    import numpy as np

    W, S = wl.window, wl.n_seq
    if n_layers > 1 and not wl.stagger:  # layer l starts its windows floor(l W / L) tokens later
        return np.repeat(((np.arange(n_layers) * W) // n_layers)[:, None], S, axis=1)
    G = W if wl.stagger else stagger_groups(wl)
    s = np.arange(S)
    if layout == "blocks" and S % G == 0:
        off = (G - 1 - s // (S // G)) * (W // G)
    else:
        off = (s % G) * (W // G)
    return np.tile(off, (n_layers, 1))


class Schedule:
    """Host mirror of the window fill of every (layer, sequence).  step()
    advances one token and returns, for each layer that needs a boundary call,
    (layer, per-sequence force mask or None, sequences due).  During the
    set-up phase (token index given) sequence s of layer l is force-flushed
    after token W - 1 - offset, so it ends the phase `offset` tokens into a
    window; later steps flush only full windows."""

    def __init__(self, wl, n_layers, layout="blocks"):
        import numpy as np

        self.W = wl.window
        self.offsets = window_offsets(wl, n_layers, layout)
        self.fill = np.zeros((n_layers, wl.n_seq), np.int64)
        self.force_at = np.where(self.offsets == 0, -1, self.W - 1 - self.offsets)

    def step(self, setup_token=None):
        self.fill += 1
        out = []
        for layer in range(self.fill.shape[0]):
            f = self.fill[layer]
            forced = (self.force_at[layer] == setup_token) if setup_token is not None else None
            due = f >= self.W
            if forced is not None:
                due = due | (forced & (f > 0))
            if due.any():
                out.append((layer, forced if (forced is not None and forced.any()) else None, int(due.sum())))
                f[due] = 0
        return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(wl, target_s, fmt="int8", buffer="fp32", single_thread_s=4.0):
    """The oracle's definitional windowed form (FP64) over one whole window of
    W decode tokens per unit, its boundary requantization included, on a
    sample of units sized to about target_s seconds on all host threads, then
    on one thread (about single_thread_s seconds)."""
    import numpy as np

    import oracle as orc
    from linear_attention_recurrent_gdn_amd import inputs as I

    src = wl.scaled(projected=False) if wl.projected else wl
    n_tok = wl.window  # one window and its boundary

    def sample(units):
        st = I.prefill_streams(src, units, n=n_tok, phase=I.PHASE_DECODE, with_queries=True)
        S0 = I.surrogate_state(src, units).astype(np.float64)
        return S0, st

    def timed(units, reps=1):
        S0, st = sample(units)
        t0 = time.perf_counter()
        for _ in range(reps):
            # the chain-free buffer computes the fp32 buffer's result
            orc.windowed_run(S0, st["q"], st["k"], st["v"], st["beta"], st["gate"], wl.window, wl.n_comp,
                             fmt=fmt, buffer="fp32" if buffer == "nform" else buffer)
        return time.perf_counter() - t0

    threads = orc.num_threads()
    cal_units = list(range(min(2 * threads, wl.n_units)))
    rate = len(cal_units) * n_tok / max(timed(cal_units), 1e-6)
    n_units = int(max(1, min(wl.n_units, rate * target_s / n_tok)))
    reps = int(max(1, min(20, round(rate * target_s / (n_units * n_tok)))))
    units = np.linspace(0, wl.n_units - 1, n_units).astype(int)
    dt = timed(units, reps)
    value = reps * n_units * n_tok / dt
    # one thread, on a smaller sample
    orc.set_num_threads(1)
    try:
        n1 = int(max(1, min(n_units, value / threads * single_thread_s / n_tok)))
        dt1 = timed(units[:n1])
    finally:
        orc.set_num_threads(threads)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except Exception:
        pass
    return {
        "value": value,
        "unit": "seq·head·tokens/s",
        "cores": threads,
        "kind": "oracle",
        "single_thread_value": n1 * n_tok / dt1,
        "sample": (f"{n_units} of {wl.n_units} units x one window of {n_tok} decode tokens with its boundary "
                   f"requantization x {reps} passes on {threads} threads ({dt:.1f} s); one thread: {n1} units, "
                   f"{dt1:.1f} s; FP64 definitional windowed form, input generation excluded; "
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


def practical_mix(units: int):
    """The access-mix probe (the decode step's reads and writes for an empty
    window, d = 128) at `units` units: GB/s for reads only, with the writes,
    and with the 512-byte writes non-temporal; None when the probe is not built."""
    import subprocess

    from linear_attention_recurrent_gdn_amd import _build

    if not os.path.exists(_build.MIX):
        return None
    r = subprocess.run([_build.MIX, str(int(units))], capture_output=True, text=True, timeout=120)
    rows = {x["mode"]: x for x in (json.loads(l) for l in r.stdout.splitlines() if l.startswith("{"))}
    if r.returncode != 0 or len(rows) != 3:
        return None
    return {name: rows[m]["TBps"] * 1e3 for m, name in ((0, "reads_only_GBps"), (1, "with_writes_GBps"),
                                                         (2, "with_writes_nt_GBps"))}


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

def timed_graph(torch, stream, body, repeats=1):
    """Capture body() as one HIP graph, replay it `repeats` times, each between
    HIP events on `stream`; the median replay time (ms)."""
    import numpy as np

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
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


def main(argv=None):
    args = parse_args(argv)
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
    W, U, L, d, H = wl.window, wl.n_units, wl.layers, wl.d, wl.n_v_heads
    K = wl.decode if args.steps is None else args.steps
    warmup = max(0, args.warmup)
    n_seg = max(1, args.repeats)
    R = max(1, args.replicas)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)  # default priority
    torch.cuda.set_stream(stream)
    gen = torch.Generator(dev).manual_seed(1000 + wl.seed)
    code_format = {"int8": lq.LQ_CODE_INT8, "e4m3": lq.LQ_CODE_E4M3}[args.format]
    buffer_format = {"fp32": lq.LQ_BUFFER_FP32, "fp16": lq.LQ_BUFFER_FP16, "nform": lq.LQ_BUFFER_NFORM}[args.buffer]
    cfg = lq.Config(wl.n_seq, wl.n_v_heads, wl.n_k_heads, d, d, W, wl.n_comp, wl.gate_kind, code_format,
                    buffer_format)
    if args.load_policy == "residency":
        in_hbm = L * R * lq.lq_state_bytes(cfg) > 2 * LLC_BYTES
        load_policy = lq.LQ_LOADS_STREAM if in_hbm else lq.LQ_LOADS_AUTO
    else:
        load_policy = {"auto": lq.LQ_LOADS_AUTO, "stream": lq.LQ_LOADS_STREAM,
                       "cached": lq.LQ_LOADS_CACHED}[args.load_policy]
    cfg = dataclasses.replace(cfg, load_policy=load_policy)
    # Boundary beside the decode (multi-layer stacks): a layer's boundary call
    # depends only on that layer's decode of the token, and only that layer's
    # decode of the next token depends on it, so it runs on a second stream
    # (default priority) with its persistent grid limited to part of the CUs
    # while the following layers decode on the rest.
    n_cus_total = torch.cuda.get_device_properties(dev).multi_processor_count
    # measured best grids (sweeps of 64-160 CUs): 96 with the fp32 buffer, 128 with
    # the binary16 one, whose shorter decode launches leave the boundary less time
    default_cus = 128 if args.buffer == "fp16" else 96
    flush_cus = args.flush_cus if args.flush_cus >= 0 else min(default_cus, n_cus_total)
    overlap = L > 1 and 0 < flush_cus
    fstream = torch.cuda.Stream(dev) if overlap else None
    cfg_side = dataclasses.replace(cfg, flush_cus=flush_cus) if overlap else cfg
    t_setup = time.perf_counter()

    # ---- start states: FP32 prefill through the FP32-state kernel (input synthesis)
    weights = [projection_weights(wl, gen, dev) for _ in range(L)] if wl.projected else [None] * L
    S_fp32, states = [], []
    o = torch.empty((wl.n_seq, H, d), device=dev)
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
    blobs = [[st] + [st.clone() for _ in range(R - 1)] for st in states]  # [layer][copy]
    if not args.no_fp32:
        S_fp32 = [[S] + [S.clone() for _ in range(R - 1)] for S in S_fp32]
    else:
        del S_fp32
    # decode inputs: a pool of tokens per layer, step t uses token t mod pool
    n_pool = min(W + warmup + n_seg * K, 32)
    pool = [device_tokens(wl, n_pool, layer, gen, dev, weights[layer]) for layer in range(L)]
    tok = lambda layer, t: pool[layer][t % n_pool]
    torch.cuda.synchronize()

    sched = Schedule(wl, L, args.stagger_layout)
    force_dev = torch.zeros(wl.n_seq, dtype=torch.uint8, device=dev)
    acct = {"decode_bytes": 0.0, "flush_bytes": 0.0, "flush_calls": 0, "flushed_units": 0, "decode_launches": 0}

    pending = [None] * L  # event of a layer's boundary call not yet waited for

    def join_flushes():
        for layer in range(L):
            if pending[layer] is not None:
                stream.wait_event(pending[layer])
                pending[layer] = None

    def q8_step(t, setup_token=None):
        side = overlap and setup_token is None
        due_now = {layer for layer in range(L) if (sched.fill[layer] + 1 >= W).any()} if side else set()
        for layer in range(L):
            if pending[layer] is not None:
                stream.wait_event(pending[layer])
                pending[layer] = None
            tk = tok(layer, t)
            fills = sched.fill[layer]
            acct["decode_bytes"] += R * H * float(sum(decode_bytes(wl, int(j)) for j in fills))
            acct["decode_launches"] += R
            for st in blobs[layer]:
                lq.lq_decode_step(cfg, st, tk["q"], tk["k"], tk["v"], tk["beta"], tk["gate"], o)
            if layer in due_now:
                ev = torch.cuda.Event()
                ev.record(stream)
                fstream.wait_event(ev)
                for st in blobs[layer]:
                    lq.lq_window_flush(cfg_side, st, None, stream=fstream)
                done = torch.cuda.Event()
                done.record(fstream)
                pending[layer] = done
        for layer, forced, n_due in sched.step(setup_token):
            if layer not in due_now:
                fm = None
                if forced is not None:
                    force_dev.copy_(torch.from_numpy(forced.astype(np.uint8)))
                    fm = force_dev
                for st in blobs[layer]:
                    lq.lq_window_flush(cfg, st, fm)
            acct["flush_calls"] += R
            acct["flushed_units"] += R * H * n_due
            acct["flush_bytes"] += R * H * n_due * flush_bytes(wl, W)

    # ---- set-up phase (window offsets), then warm-up: untimed
    for t in range(W):
        q8_step(t, setup_token=t)
    assert (sched.fill == sched.offsets).all()
    for t in range(W, W + warmup):
        q8_step(t)
    join_flushes()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    # ---- timed: n_seg consecutive segments of K steps, one graph each, replayed once
    for key in acct:
        acct[key] = 0
    t0 = W + warmup
    seg_ms = []
    for r in range(n_seg):
        a = t0 + r * K
        seg_ms.append(timed_graph(torch, stream, lambda: ([q8_step(t) for t in range(a, a + K)], join_flushes())))
    ms_seg = float(np.median(seg_ms))
    flags = [lq.lq_read_status(cfg, st) for bl in blobs for st in bl]
    if any(flags):
        raise RuntimeError(f"device flags set during the run: {flags}")
    steps_timed = n_seg * K
    units_step = U * L * R
    ws_bytes = L * R * lq.lq_state_bytes(cfg)
    result = {
        "metric": METRIC,
        "value": units_step * K / (ms_seg * 1e-3),
        "unit": "seq·head·tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": ms_seg / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "state_dtype": args.format,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "layers": L, "n_seq": wl.n_seq, "n_v_heads": H, "n_k_heads": wl.n_k_heads,
            "d_k": d, "d_v": d, "gate": wl.gate, "window": W, "n_comp": wl.n_comp,
            "code_format": args.format, "buffer_format": args.buffer,
            "prefill": wl.prefill, "units": units_step, "state_copies": R,
            "state_bytes": ws_bytes,
            "load_policy": {lq.LQ_LOADS_AUTO: "auto", lq.LQ_LOADS_STREAM: "stream",
                            lq.LQ_LOADS_CACHED: "cached"}[cfg.load_policy],
            "residency": ("hbm" if ws_bytes > 2 * LLC_BYTES else
                          "cache (the states fit the 256 MB last-level cache; --replicas pushes them to HBM)"),
        },
        "timing": (f"{n_seg} consecutive segments of {K} steps after {W} set-up and {warmup} warm-up steps; "
                   f"each segment one HIP graph replayed once between HIP events; median segment "
                   f"({', '.join(f'{x:.3f}' for x in seg_ms)} ms); windows staggered "
                   + (f"per sequence (the workload's offsets, {W} groups, layout {args.stagger_layout})"
                      if wl.stagger else
                      f"across layers (layer l offset floor(l*{W}/{L}))" if L > 1 else
                      f"over {stagger_groups(wl)} sequence groups (layout {args.stagger_layout})")
                   + ", so the timed steps carry their share of boundary requantization"
                   + (f"; each layer's boundary call on a second stream with its grid on {flush_cus} of "
                      f"{n_cus_total} CUs, beside the next layers' decode steps (that layer's next decode waits "
                      f"for it; every segment ends when its last boundary call has)" if overlap else
                      "; boundary calls on the decode stream")),
        "boundary_stream": ({"flush_cus": flush_cus, "of": n_cus_total, "overlapped": True} if overlap else
                            {"overlapped": False}),
        "timed_steps": {
            "decode_launches": acct["decode_launches"],
            "flush_calls": acct["flush_calls"],
            "flushed_units": acct["flushed_units"],
            "flushed_units_per_step": acct["flushed_units"] / steps_timed,
            "flush_share_expected_per_step": units_step / W,
            "alg_bytes_per_step": (acct["decode_bytes"] + acct["flush_bytes"]) / steps_timed,
            "alg_GBps": (acct["decode_bytes"] + acct["flush_bytes"]) / steps_timed / (ms_seg / K * 1e-3) / 1e9,
        },
        "setup_s": round(setup_s, 1),
    }

    # ---- FP32-state comparison on the same steps
    fp32 = None
    if not args.no_fp32:
        def fp32_steps(ta, tb):
            for t in range(ta, tb):
                for layer in range(L):
                    tk = tok(layer, t)
                    for S in S_fp32[layer]:
                        lq.lq_fp32_decode_step(cfg, S, tk["q"], tk["k"], tk["v"], tk["beta"], tk["gate"], o)
        fp32_steps(0, warmup)
        fp32_ms = timed_graph(torch, stream, lambda: fp32_steps(t0, t0 + K), n_seg)
        g = d if wl.gate == "channel" else 1
        fp32_b = 8 * d * d + 4 * (2 * d // wl.group + 2 * d + 1 + g)
        fp32 = {
            "value": units_step * K / (fp32_ms * 1e-3),
            "ms_per_step": fp32_ms / K,
            "alg_GBps": units_step * fp32_b / (fp32_ms / K * 1e-3) / 1e9,
            "speedup_vs_fp32": fp32_ms / ms_seg,
        }
        result["fp32_state"] = fp32
        del S_fp32

    # ---- the decode kernel alone over one whole window (every layer at fill
    # 0 .. W-1), as one graph: its average launch time against its bytes
    all_seq = torch.ones(wl.n_seq, dtype=torch.uint8, device=dev)
    for bl in blobs:
        for st in bl:
            lq.lq_window_flush(cfg, st, all_seq)  # forced: every window restarts empty
    dec_ms = timed_graph(torch, stream, lambda: [lq.lq_decode_step(cfg, st, tok(layer, j)["q"], tok(layer, j)["k"],
                                                                    tok(layer, j)["v"], tok(layer, j)["beta"],
                                                                    tok(layer, j)["gate"], o)
                                                  for j in range(W) for layer in range(L) for st in blobs[layer]])
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
        "note": "one graph of one window of decode launches (every layer and copy at j = 0..W-1), HIP events "
                "around the replay on the launch stream; bytes = the mean over j of the per-unit model x units",
    }
    # ---- the boundary kernel alone: every unit of a layer after a full window
    fl_ms = timed_graph(torch, stream, lambda: [lq.lq_window_flush(cfg, blobs[layer][0], None) for layer in range(L)])
    fl_s = fl_ms * 1e-3 / L
    flops = 5.0 * d * d * W * U
    result["flush"] = {
        "avg_launch_us": fl_s * 1e6,
        "units_per_launch": U,
        "tokens_replayed": W,
        "alg_GBps": flush_bytes(wl, W) * U / fl_s / 1e9,
        "roofline": {"bound": "mfma", "achieved": flops / fl_s / 1e12, "peak": PEAK_FP64_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / fl_s / 1e12 / PEAK_FP64_MFMA_TFLOPS,
                     "dtype": "f64", "flops_per_unit": 5.0 * d * d * W,
                     "kernel": "materialize_kernel (flush mode) + due_scan_kernel",
                     "note": "5 d^2 W flop per unit (the window transform's products); one launch per layer "
                             "over all its units, HIP events around a graph of the layers' launches"},
    }

    # ---- self-checks
    dec_floor_ms = L * R * avg_launch_s * 1e3
    checks = {
        "decode_launches_ms_per_step": dec_floor_ms,
        "ms_per_step_over_decode_launches": (ms_seg / K) / dec_floor_ms,
        "ms_per_step_at_least_decode_launches": bool(ms_seg / K >= 0.97 * dec_floor_ms),
        # the boundary work per step if its time scaled with the units flushed
        "flush_model_ms_per_step": (acct["flushed_units"] / steps_timed) / U * fl_s * 1e3,
    }
    # with the boundary beside the decode: the part of (decode launches +
    # boundary model) that the step no longer pays
    checks["boundary_hidden_ms_per_step"] = (dec_floor_ms + checks["flush_model_ms_per_step"]) - ms_seg / K
    if fp32 is not None:
        int8_b = result["timed_steps"]["alg_bytes_per_step"]
        g = d if wl.gate == "channel" else 1
        fp32_step_b = units_step * (8 * d * d + 4 * (2 * d // wl.group + 2 * d + 1 + g))
        ceiling = fp32_step_b / int8_b
        checks["byte_ratio_ceiling"] = ceiling
        checks["speedup_over_ceiling"] = fp32["speedup_vs_fp32"] / ceiling
    result["checks"] = checks

    if not args.no_prefill and wl.prefill > 0 and not wl.projected and L == 1 and R == 1:
        result["prefill"] = prefill_timing(lq, wl, cfg, gen, dev,
                                           lambda body, reps=1: timed_graph(torch, stream, body, reps))

    # the practical ceiling at the decode launch's byte count (a child process;
    # the device is idle here)
    torch.cuda.synchronize()
    pr = practical_read(avg_bytes)
    if pr is not None:
        result["roofline"]["practical"] = {
            "kernel": "stream_read (probe/stream_read.hip): 16-byte loads, grid-stride, nothing else; "
                      "consecutive launches read disjoint regions of a >= 2 GiB pool (HBM, not the cache)",
            "bytes_per_launch": avg_bytes, "achieved": pr["GBps"], "unit": "GB/s",
            "frac_of_peak": pr["GBps"] / HBM_PEAK_GBS, "decode_frac_of_practical": achieved / pr["GBps"],
        }

    if d == 128:
        pm = practical_mix(U)
        if pm is not None:
            result["roofline"]["practical_mix"] = dict(
                kernel="access_mix (probe/access_mix.hip): the decode step's reads and writes for an empty window, "
                       "nothing else, at this launch's unit count", unit="GB/s", **pm)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, args.format, args.buffer)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
