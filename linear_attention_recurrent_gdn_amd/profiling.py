"""Measurement helpers around rocprofv3 (no part of the decode path).

Three commands:

  window   --workload W [--format int8|e4m3] [--buffer fp32|fp16]
      Runs, eagerly on cuda:0, one plain device-to-device copy of COPY_BYTES
      (the calibration kernel for the memory counters), then one whole window
      of decode launches (every unit at fill j = 0 .. W-1) on a freshly
      initialised state.  Meant to run under ``rocprofv3 --pmc FETCH_SIZE``
      and, in a second run, ``--pmc WRITE_SIZE``.

  traffic  --workload W --fetch DIR --write DIR --out FILE
      Reads the two counter_collection.csv files, scales the decode kernel's
      per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) by the factor that makes the
      copy read and write exactly COPY_BYTES, and writes the per-launch HBM
      bytes averaged over the window, keyed by a hash of the decode kernel's
      source (a changed kernel invalidates the figure).

  stats    --csv FILE --cmd "..." --out FILE
      Formats a ``rocprofv3 --stats`` kernel_stats.csv as a short text
      summary headed by the command that produced it.

  flush    --workload W [--launches N]
      Runs N window-boundary launches on one layer of the workload's shape
      (every unit's window filled by W decode launches first, synthetic
      tokens), meant to run under ``rocprofv3 --pmc SQ_INSTS_MFMA
      SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE``.

  mfma     --workload W --dir DIR --out FILE --command "..."
      Reads that run's counter_collection.csv and writes, per flush launch,
      the matrix-core counters, the busy fraction of the matrix pipes and the
      FP64 rate the instruction count implies.

  overlap  --trace FILE --out FILE --command "..."
      Reads a kernel_trace.csv of the stack benchmark (boundary calls on a
      second stream beside the next layers' decode steps) and writes: the
      boundary dispatches that ran beside decode launches (count, grid in
      workgroups, mean duration) against those that ran alone, and, between
      the first and the last of the former, the decode launches that ran beside
      a boundary against those that did not (count, mean duration).

  hbm
      Practical memory bandwidth of this device for plain streaming kernels:
      the stream_read yardstick (probe/stream_read.hip: 16-byte loads,
      grid-stride, nothing else) over the decode launches' own byte counts
      (56.4 MB, 379 MB, 506 MB and 902 MB per launch for gdn_decode,
      hybrid_stack, kda_decode and gdn_serving) and 4 GiB, then torch's 1 GiB
      device-to-device copy (read + write) and read (sum) and the same over
      64 MiB; every figure timed with HIP events over repeated launches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
DECODE_KERNEL = "decode_q8_kernel"
COPY_KERNEL = "copyBuffer"


def kernel_sha() -> str:
    """Short hash of the decode kernel's source file."""
    with open(os.path.join(HERE, "csrc", "lq_decode.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def run_window(workload: str, fmt: str = "int8", buffer: str = "fp32") -> None:
    import torch

    import linear_attention_recurrent_gdn_amd as lq
    from linear_attention_recurrent_gdn_amd import inputs as I

    lq.load_library()
    wl = I.WORKLOADS[workload]
    U, d, W = wl.n_units, wl.d, wl.window
    dev = torch.device("cuda", 0)
    gen = torch.Generator(dev).manual_seed(2000 + wl.seed)
    code_format = {"int8": lq.LQ_CODE_INT8, "e4m3": lq.LQ_CODE_E4M3}[fmt]
    buffer_format = {"fp32": lq.LQ_BUFFER_FP32, "fp16": lq.LQ_BUFFER_FP16}[buffer]
    cfg = lq.Config(wl.n_seq, wl.n_v_heads, wl.n_k_heads, d, d, W, wl.n_comp, wl.gate_kind, code_format,
                    buffer_format)

    src = torch.empty(COPY_BYTES // 4, device=dev).normal_(generator=gen)
    dst = torch.empty_like(src)
    state = lq.new_state(cfg, dev)
    S0 = torch.randn((U, d, d), generator=gen, device=dev) * 0.5
    lq.lq_state_init(cfg, state, S0)
    del S0
    if wl.projected:
        from bench import projected, projection_weights  # input synthesis only

        w = projection_weights(wl, gen, dev)
        toks = [projected(wl, w, torch.randn((wl.n_seq, wl.hidden), generator=gen, device=dev)
                          .to(torch.bfloat16)) for _ in range(W)]
    else:
        toks = [I.torch_token(wl, gen, dev) for _ in range(W)]
    o = torch.empty((wl.n_seq, wl.n_v_heads, d), device=dev)
    torch.cuda.synchronize()
    print(f"[window] {workload}: copy of {COPY_BYTES} B", flush=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[window] {workload}: {W} decode launches over {U} units", flush=True)
    for t in range(W):
        tk = toks[t]
        lq.lq_decode_step(cfg, state, tk["q"], tk["k"], tk["v"], tk["beta"], tk["gate"], o)
    torch.cuda.synchronize()
    flags = lq.lq_read_status(cfg, state)
    print(f"[window] done, flags={flags:#x}", flush=True)
    if flags:
        sys.exit(1)


def run_flush(workload: str, launches: int = 3) -> None:
    import torch

    import linear_attention_recurrent_gdn_amd as lq
    from linear_attention_recurrent_gdn_amd import inputs as I

    lq.load_library()
    wl = I.WORKLOADS[workload].scaled(projected=False, layers=1)
    U, d, W = wl.n_units, wl.d, wl.window
    dev = torch.device("cuda", 0)
    gen = torch.Generator(dev).manual_seed(3000 + wl.seed)
    cfg = lq.Config(wl.n_seq, wl.n_v_heads, wl.n_k_heads, d, d, W, wl.n_comp, wl.gate_kind)
    state = lq.new_state(cfg, dev)
    S0 = torch.randn((U, d, d), generator=gen, device=dev) * 0.5
    lq.lq_state_init(cfg, state, S0)
    del S0
    toks = [I.torch_token(wl, gen, dev) for _ in range(min(W, 16))]
    o = torch.empty((wl.n_seq, wl.n_v_heads, d), device=dev)
    for n in range(launches):
        for t in range(W):
            tk = toks[t % len(toks)]
            lq.lq_decode_step(cfg, state, tk["q"], tk["k"], tk["v"], tk["beta"], tk["gate"], o)
        torch.cuda.synchronize()
        print(f"[flush] {workload}: boundary {n + 1}/{launches} over {U} units, {W} tokens each", flush=True)
        lq.lq_window_flush(cfg, state, None)
        torch.cuda.synchronize()
    flags = lq.lq_read_status(cfg, state)
    print(f"[flush] done, flags={flags:#x}", flush=True)
    if flags:
        sys.exit(1)


MFMA_F64_FLOP = 2 * 16 * 16 * 4  # one v_mfma_f64_16x16x4f64
PEAK_FP64_TFLOPS = 78.6
N_CU = 256


def mfma(workload: str, directory: str, out: str, cmd: str) -> dict:
    """Per flush launch: the matrix-core counters and what they imply."""
    from linear_attention_recurrent_gdn_amd import inputs as I

    wl = I.WORKLOADS[workload]
    cnt = {}
    for name in ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"):
        cnt[name] = _per_dispatch(_counter_rows(directory, name), "materialize_kernel")
    n = len(cnt["SQ_INSTS_MFMA"])
    if n == 0 or any(len(v) != n for v in cnt.values()):
        raise SystemExit(f"expected the same flush dispatches for every counter, found "
                         f"{ {k: len(v) for k, v in cnt.items()} }")
    rows = []
    for i in range(n):
        mf, busy, sqb, gui = (cnt[k][i] for k in ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
                                                  "GRBM_GUI_ACTIVE"))
        rows.append({"mfma_insts": mf, "mfma_busy_cycles": busy, "sq_busy_cycles": sqb, "gui_active": gui,
                     "busy_cycles_per_mfma": busy / mf if mf else 0.0,
                     "mfma_flop": mf * MFMA_F64_FLOP})
    rec = {"kernel": "materialize_kernel (flush mode)", "workload": workload, "units": wl.n_units,
           "window": wl.window, "dispatches": rows, "command": cmd}
    lines = [f"# matrix-core counters of the window-boundary kernel, {workload} shape "
             f"({wl.n_units} units, W = {wl.window}, d = {wl.d})",
             f"# command: {cmd}", "#",
             "# per dispatch of the materialize kernel (the first is the state init, which replays nothing; "
             "then the boundaries): SQ_INSTS_MFMA, SQ_VALU_MFMA_BUSY_CYCLES, busy cycles per MFMA, "
             "GRBM_GUI_ACTIVE, MFMA flop (16x16x4 FP64: 2048 each), SQ_BUSY_CYCLES, matrix-pipe busy fraction "
             "(busy cycles / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs))"]
    for r in rows:
        frac = r["mfma_busy_cycles"] / (r["gui_active"] / 8.0 * 4 * N_CU) if r["gui_active"] else 0.0
        kind = "boundary" if r["mfma_insts"] else "init"
        lines.append(f"  {kind:8s} {r['mfma_insts']:14.0f} {r['mfma_busy_cycles']:16.0f} {r['busy_cycles_per_mfma']:7.2f} "
                     f"{r['gui_active']:14.0f} {r['mfma_flop']:16.4g} {r['sq_busy_cycles']:14.0f} {frac:6.3f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rec


STREAM_BYTES = (56397824, 378830848, 505602048, 902365184, 4 << 30)
MIX_UNITS = (1024, 4096, 8192, 16384)  # decode launch sizes of the workloads


def hbm() -> dict:
    import subprocess

    from linear_attention_recurrent_gdn_amd import _build

    if not os.path.exists(_build.PROBE):
        raise SystemExit(f"{_build.PROBE} is missing: build it first (python -m linear_attention_recurrent_gdn_amd._build)")
    r = subprocess.run([_build.PROBE, *map(str, STREAM_BYTES)], capture_output=True, text=True)
    sys.stdout.write(r.stdout)
    if r.returncode != 0:
        raise SystemExit(f"stream_read failed: {r.stderr.strip()}")
    out = {"stream_read": [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]}
    out["access_mix"] = []
    if os.path.exists(_build.MIX):
        for units in MIX_UNITS:
            r = subprocess.run([_build.MIX, str(units)], capture_output=True, text=True)
            sys.stdout.write(r.stdout)
            if r.returncode != 0:
                raise SystemExit(f"access_mix failed: {r.stderr.strip()}")
            out["access_mix"] += [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    import torch

    dev = torch.device("cuda", 0)
    for label, nbytes in (("1GiB", 1 << 30), ("64MiB", 64 << 20)):
        x = torch.ones(nbytes // 4, device=dev)
        y = torch.empty_like(x)
        for kind in ("copy", "read"):
            def body():
                return y.copy_(x) if kind == "copy" else x.sum()
            for _ in range(3):
                body()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 20
            a.record()
            for _ in range(reps):
                body()
            b.record()
            torch.cuda.synchronize()
            sec = a.elapsed_time(b) * 1e-3 / reps
            moved = nbytes * (2 if kind == "copy" else 1)
            out[f"{kind}_{label}_TBps"] = round(moved / sec / 1e12, 3)
        del x, y
    print(json.dumps(out))
    return out


def _counter_rows(path_or_dir: str, counter: str):
    paths = [path_or_dir] if os.path.isfile(path_or_dir) else \
        glob.glob(os.path.join(path_or_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {path_or_dir}")
    rows = []
    for p in paths:
        with open(p) as f:
            rows += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    return rows


def _per_dispatch(rows, name_part):
    by = {}
    for r in rows:
        if name_part in r["Kernel_Name"]:
            key = int(r["Dispatch_Id"])
            by[key] = by.get(key, 0.0) + float(r["Counter_Value"])
    return [by[k] for k in sorted(by)]


def traffic(workload: str, fetch_dir: str, write_dir: str, out: str, cmd: str) -> dict:
    from linear_attention_recurrent_gdn_amd import inputs as I

    wl = I.WORKLOADS[workload]
    res = {}
    for tag, counter, path in (("fetch", "FETCH_SIZE", fetch_dir), ("write", "WRITE_SIZE", write_dir)):
        rows = _counter_rows(path, counter)
        # the runtime's own small copies (status reads) use the same blit kernel:
        # the calibration copy is the largest one
        copy = max(_per_dispatch(rows, COPY_KERNEL), default=0.0)
        dec = _per_dispatch(rows, DECODE_KERNEL)
        if copy <= 0 or len(dec) != wl.window:
            raise SystemExit(f"{counter}: expected a copy and {wl.window} decode dispatches, "
                             f"found copy={copy} and {len(dec)}")
        factor = (COPY_BYTES / 1024.0) / copy
        res[tag] = {"copy_kib": copy, "factor": factor,
                    "decode_kib_per_launch_raw": sum(dec) / len(dec),
                    "decode_bytes_per_launch": factor * 1024.0 * sum(dec) / len(dec),
                    "first_last_kib_raw": [dec[0], dec[-1]]}
    rec = {
        "kernel": DECODE_KERNEL,
        "workload": workload,
        "kernel_sha": kernel_sha(),
        "launches": wl.window,
        "hbm_bytes_per_launch": res["fetch"]["decode_bytes_per_launch"] + res["write"]["decode_bytes_per_launch"],
        "fetch": res["fetch"],
        "write": res["write"],
        "calibration": f"one device copy of {COPY_BYTES} B read and written in the same run",
        "command": cmd,
    }
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def tail_mean_us(trace_csv: str, name_part: str, n: int):
    """Mean duration (us) of the last n dispatches of a kernel in a kernel trace."""
    with open(trace_csv) as f:
        rows = [r for r in csv.DictReader(f) if name_part in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    tail = rows[-n:]
    if not tail:
        return None
    return sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tail) / len(tail) / 1e3, len(tail)


def stats(csv_path: str, cmd: str, out: str, trace_csv: str = None, tail_kernel: str = None,
          tail_n: int = 0) -> None:
    with open(csv_path) as f:
        rows = list(csv.DictReader(f))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {cmd}", "#",
             f"# {'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10} {'pct':>6}  kernel"]
    for r in rows:
        name = r["Name"]
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"  {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['TotalDurationNs']) / 1e6:10.3f} "
                     f"{float(r['Percentage']):6.2f}  {name}")
    if trace_csv and tail_kernel and tail_n > 0:
        res = tail_mean_us(trace_csv, tail_kernel, tail_n)
        if res is not None:
            mean, n = res
            lines.append("#")
            lines.append(f"# {tail_kernel}: mean of its last {n} dispatches (the benchmark's graph of one "
                         f"window of decode launches): {mean:.2f} us")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    print(text)


def overlap(trace_csv: str, cmd: str, out: str) -> str:
    """Boundary dispatches beside decode launches, and decode launches beside
    a boundary, from one kernel trace (times in us)."""
    dec, flu = [], []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            span = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
            if DECODE_KERNEL in name:
                dec.append(span)
            elif "materialize_kernel<" in name and name.split("<")[1].split(",")[2].strip() == "1":
                wg = int(r["Workgroup_Size_X"])
                flu.append(span + (int(r["Grid_Size_X"]) // max(wg, 1),))
    dec.sort()
    flu.sort()
    starts = [s for s, _ in dec]

    import bisect

    def beside(a, b):  # decode launches overlapping [a, b)
        i = bisect.bisect_left(starts, a) - 1
        i = max(i, 0)
        out_ = []
        while i < len(dec) and dec[i][0] < b:
            if dec[i][1] > a:
                out_.append(i)
            i += 1
        return out_

    with_dec, alone = [], []
    overlapped_dec = set()
    for s, e, g in flu:
        idx = beside(s, e)
        (with_dec if idx else alone).append((s, e, g))
        overlapped_dec.update(idx)
    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    lines = ["# window-boundary kernel beside the decode (kernel trace)", f"# command: {cmd}", "#"]
    lines.append(f"# boundary dispatches beside decode launches: {len(with_dec)}, grid "
                 f"{sorted(set(g for _, _, g in with_dec))} workgroups, mean "
                 f"{mean([(e - s) / 1e3 for s, e, _ in with_dec]):.1f} us")
    lines.append(f"# boundary dispatches alone: {len(alone)}, grid {sorted(set(g for _, _, g in alone))} "
                 f"workgroups, mean {mean([(e - s) / 1e3 for s, e, _ in alone]):.1f} us")
    if with_dec:
        a, b = with_dec[0][0], with_dec[-1][1]
        region = [i for i in range(len(dec)) if a <= dec[i][0] < b]
        bd = [(dec[i][1] - dec[i][0]) / 1e3 for i in region if i in overlapped_dec]
        al = [(dec[i][1] - dec[i][0]) / 1e3 for i in region if i not in overlapped_dec]
        lines.append(f"# decode launches in that span: {len(region)}; beside a boundary {len(bd)}, mean "
                     f"{mean(bd):.2f} us; alone {len(al)}, mean {mean(al):.2f} us")
        lines.append("# (the two groups mix window fills in different proportions: compare launches of the "
                     "same layer and fill for the slowdown itself)")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    print(text)
    return text


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("window")
    a.add_argument("--workload", default="gdn_decode")
    a.add_argument("--format", default="int8", choices=("int8", "e4m3"))
    a.add_argument("--buffer", default="fp32", choices=("fp32", "fp16"))
    b = sub.add_parser("traffic")
    b.add_argument("--workload", default="gdn_decode")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--out", required=True)
    b.add_argument("--command", default="")
    h = sub.add_parser("hbm")
    h.add_argument("--out", default=None, help="also write a text summary here")
    c = sub.add_parser("stats")
    c.add_argument("--csv", required=True)
    c.add_argument("--command", default="")
    c.add_argument("--out", required=True)
    c.add_argument("--trace", default=None, help="kernel_trace.csv of the same run")
    c.add_argument("--tail-kernel", default=None)
    c.add_argument("--tail", type=int, default=0, help="also report the mean of the kernel's last N dispatches")
    fl = sub.add_parser("flush")
    fl.add_argument("--workload", default="gdn_decode")
    fl.add_argument("--launches", type=int, default=3)
    ov = sub.add_parser("overlap")
    ov.add_argument("--trace", required=True)
    ov.add_argument("--out", required=True)
    ov.add_argument("--command", default="")
    m = sub.add_parser("mfma")
    m.add_argument("--workload", default="gdn_decode")
    m.add_argument("--dir", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--command", default="")
    args = ap.parse_args(argv)
    if args.cmd == "window":
        run_window(args.workload, args.format, args.buffer)
    elif args.cmd == "hbm":
        res = hbm()
        if args.out:
            lines = ["# streaming bandwidth of this device (plain kernels, HIP events)",
                     "# command: python -m linear_attention_recurrent_gdn_amd.profiling hbm --out " + args.out,
                     "#", "# stream_read (probe/stream_read.hip): bytes read per launch, grid, mean us, TB/s"]
            for r in res["stream_read"]:
                lines.append(f"  {r['bytes']:>12d} {r['grid']:6d} {r['us']:10.2f} {r['TBps']:7.3f}")
            lines.append("#")
            lines.append("# access_mix (probe/access_mix.hip): the decode step's accesses for an empty window "
                         "(d = 128, 4 compensators, 2 value heads per key head);")
            lines.append("# mode 0 reads only, 1 with its writes, 2 with the 512-byte writes non-temporal")
            lines.append("# units, mode, mean us, MB read, MB written, TB/s")
            for r in res.get("access_mix", []):
                lines.append(f"  {r['units']:>7d} {r['mode']:4d} {r['us']:10.2f} {r['read_bytes'] / 1e6:9.1f} "
                             f"{r['write_bytes'] / 1e6:8.2f} {r['TBps']:7.3f}")
            lines.append("# torch: " + ", ".join(f"{k} {v}" for k, v in res.items()
                                                 if k not in ("stream_read", "access_mix")))
            with open(args.out, "w") as f:
                f.write("\n".join(lines) + "\n")
    elif args.cmd == "traffic":
        print(json.dumps(traffic(args.workload, args.fetch, args.write, args.out, args.command), indent=1))
    elif args.cmd == "flush":
        run_flush(args.workload, args.launches)
    elif args.cmd == "overlap":
        overlap(args.trace, args.command, args.out)
    elif args.cmd == "mfma":
        print(json.dumps(mfma(args.workload, args.dir, args.out, args.command), indent=1))
    else:
        stats(args.csv, args.command, args.out, args.trace, args.tail_kernel, args.tail)


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(HERE))
    main()
