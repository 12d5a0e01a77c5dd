"""Benchmark of the three-tier activation-sparse decode path on one MI355X.

Workload: 7B-shaped attention projections (q, k, v, o, each 4096 x 4096,
fp16 weights ~ N(0, 0.02), column-major) with an int4 group-128 compressed
copy, tiers skip / approx / full = 40 / 30 / 30 % of the 4096 inputs, batch 1,
32 decode tokens of fresh Laplace(0, 1) activations per step.

One step = the whole per-token path for 32 tokens, through spax_layer_step:
    rank h -> tier lists -> tiered product of q, k, v (rows stacked)
    rank z -> tier lists -> tiered product of o
(each group is one fused launch: the ranking runs inside the product).
Token t reads weight set t (32 distinct sets = 32 decoder layers' attention
weights, 5.4 GB), so a set is read again only after the other 31 have
streamed through, as in decoding a 32-layer model: weights come from HBM,
not from the 256 MB last-level cache.

The step is captured once in a HIP graph (through torch's graph capture on
the stream the library launches on) and replayed; warmup replays are
untimed, then exactly --steps replays are timed between two device
synchronisations. Inputs are resident in HBM before timing starts.

Printed: ONE JSON line with the throughput (effective weight GB/s on the
algorithmic bytes), microseconds per tiered projection, the roofline of the
tiered product kernel (event-timed per launch on the launch stream) and the
CPU oracle timed on a bounded sample of the same workload. The per-launch
duration of the product kernel comes from graph replays of one group's 32
launches back to back, timed with events on the launch stream.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--eager]
                    [--no-cpu-baseline] [--calib-copy]
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

METRIC = ("µs per tiered projection & effective weight GB/s (% of HBM peak), "
          "batch-1 decode")
HBM_PEAK_GBS = 8000.0
HIDDEN = 4096
TOKENS = 32
SETS = 32
CONFIG_ID = 2


PMC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_kernel_7b_attention_pmc.txt")
KERNEL_SOURCES = ("gemv.hip", "api.cpp", "spax_internal.h")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "activation_sparse_decode_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the product kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's reading),
    or None when the kernel sources changed since the counters were taken."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:"):
            vals["traffic"] = float(line.split(":", 1)[1])
        elif line.startswith("kernel sources sha256"):
            vals["sha"] = line.rsplit(":", 1)[1].strip()
    if vals.get("sha") != kernel_source_hash() or "traffic" not in vals:
        return None
    return int(vals["traffic"])


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--sets", type=int, default=SETS,
                   help="distinct weight sets rotated over the tokens (default 32)")
    p.add_argument("--eager", action="store_true",
                   help="launch every kernel from Python instead of replaying a graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one plain 256 MiB device copy (counter calibration)")
    return p.parse_args()


class Workload:
    """Device-resident weights, inputs, outputs and lists of one step."""

    def __init__(self, sets: int):
        import torch

        import activation_sparse_decode_token_amd as spax
        import workloads as WL
        from activation_sparse_decode_token_amd.layouts import build_matrix

        self.spax = spax
        dev = torch.device("cuda:0")
        split = WL.CONFIGS[CONFIG_ID].splits[0]
        self.kf, self.ka = WL.tier_counts(HIDDEN, split)
        self.sets = sets
        ks = ([self.kf, self.kf, 0, 0], [self.ka, self.ka, 0, 0])
        self.layers, self.qkv_only, self.o_only = [], [], []
        for s in range(sets):
            q, k, v, o = (WL.weights_fp16_torch(CONFIG_ID, s, m, HIDDEN, HIDDEN, 0.02, dev)
                          for m in ("q", "k", "v", "o"))
            stacked = torch.cat([q, k, v], dim=1).contiguous()     # [n, 3*4096]
            del q, k, v
            Wqkv = build_matrix(stacked, spax.FMT_FP16, spax.FMT_INT4_G128)
            Wo = build_matrix(o, spax.FMT_FP16, spax.FMT_INT4_G128)
            del stacked, o
            # the attention groups of one decoder layer: rank h -> q, k, v;
            # rank z -> o (SpAx page, section 5.2 step 1 groups)
            self.layers.append(spax.Layer.make([Wqkv, Wo, None, None], *ks))
            self.qkv_only.append(spax.Layer.make([Wqkv, None, None, None], *ks))
            self.o_only.append(spax.Layer.make([None, Wo, None, None], *ks))
        torch.cuda.synchronize()
        f16, i32 = torch.float16, torch.int32
        self.io = []
        for t in range(TOKENS):
            h = WL.laplace_fp16_torch(CONFIG_ID, 0, "h", t, HIDDEN, dev)
            z = WL.laplace_fp16_torch(CONFIG_ID, 0, "z", t, HIDDEN, dev)
            F = [torch.empty(self.kf, dtype=i32, device=dev) for _ in range(2)]
            A = [torch.empty(self.ka, dtype=i32, device=dev) for _ in range(2)]
            self.io.append(spax.LayerIO.make(
                h=h, z=z, qkv=torch.empty(3 * HIDDEN, dtype=f16, device=dev),
                o=torch.empty(HIDDEN, dtype=f16, device=dev),
                full_idx=(F[0], F[1], None, None), approx_idx=(A[0], A[1], None, None)))
        wsb = spax.layer_workspace_bytes(self.layers[0])
        self.ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
        self.ws_bytes = wsb
        torch.cuda.synchronize()

    # bytes the method must move (selected columns, codes and scales, x,
    # index lists, y) -- see workloads.accounting
    def gemv_bytes(self):
        from workloads.accounting import gemv_algorithmic_bytes
        qkv = gemv_algorithmic_bytes(3 * HIDDEN, HIDDEN, self.kf, self.ka, "fp16", "int4")
        o = gemv_algorithmic_bytes(HIDDEN, HIDDEN, self.kf, self.ka, "fp16", "int4")
        return qkv, o

    def step_bytes(self):
        qkv, o = self.gemv_bytes()
        return TOKENS * (qkv + o)

    def step(self, stream=None):
        """Enqueue one step: every token runs the attention groups of the
        layer whose weights it reads (one fused launch per group)."""
        spax = self.spax
        for t in range(TOKENS):
            spax.layer_step(self.layers[t % self.sets], self.io[t], self.ws, self.ws_bytes,
                            compute_stream=stream)

    def launches(self, group: int):
        """The product launches of one group (0: q,k,v; 1: o) for every
        token, enqueued back to back -- one fused launch each."""
        spax = self.spax
        layers = self.qkv_only if group == 0 else self.o_only

        def run(stream):
            for t in range(TOKENS):
                spax.layer_step(layers[t % self.sets], self.io[t], self.ws, self.ws_bytes,
                                compute_stream=stream)
        return run


def graph_launch_time(run, stream, launches: int, reps: int = 5) -> float:
    """Average duration (s) of one launch: `run` (launches kernels back to
    back) is captured in a HIP graph, replayed `reps` times between two
    events on the launch stream."""
    import torch
    with torch.cuda.stream(stream):
        run(stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run(stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (reps * launches)


def gpu_run(args):
    import torch

    import activation_sparse_decode_token_amd as spax
    spax.lib()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (torch.cuda.is_available() is False)")
    log(f"device {torch.cuda.get_device_name(0)}; building {args.sets} weight sets")
    t0 = time.perf_counter()
    wl = Workload(args.sets)
    log(f"weights ready in {time.perf_counter() - t0:.1f} s; "
        f"k_full={wl.kf} k_approx={wl.ka}")

    stream = torch.cuda.Stream()
    graph = None
    with torch.cuda.stream(stream):
        wl.step(stream)                      # eager warm pass (also loads code objects)
        torch.cuda.synchronize()
        if not args.eager:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                wl.step(stream)
            torch.cuda.synchronize()

    def run_once():
        if graph is not None:
            graph.replay()
        else:
            wl.step(stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run_once()
        torch.cuda.synchronize()
        log(f"warmup done ({args.warmup} steps, {'eager' if graph is None else 'graph'})")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            run_once()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_event = ev0.elapsed_time(ev1)
    log(f"timed {args.steps} steps: wall {wall * 1e3:.2f} ms, events {ms_event:.2f} ms")

    # Per-launch duration of the product kernel, event-timed on its stream:
    # each group's launches back to back in a graph (host launch cost is
    # not on the GPU timeline).
    qkv_b, o_b = wl.gemv_bytes()
    if graph is not None:
        t_qkv = graph_launch_time(wl.launches(0), stream, TOKENS)
        t_o = graph_launch_time(wl.launches(1), stream, TOKENS)
        avg_us = (t_qkv + t_o) / 2 * 1e6
        achieved = (qkv_b + o_b) / (t_qkv + t_o) / 1e9
        log(f"product kernel: qkv {t_qkv * 1e6:.2f} us, o {t_o * 1e6:.2f} us per launch, "
            f"{achieved:.0f} GB/s on algorithmic bytes")
    else:
        t_qkv = t_o = avg_us = achieved = None
    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy: 268435456 bytes read, 268435456 bytes written")

    sec_step = ms_event * 1e-3 / args.steps
    step_b = wl.step_bytes()
    return {
        "sec_step": sec_step,
        "wall_step": wall / args.steps,
        "step_bytes": step_b,
        "projections": TOKENS * 4,
        "roofline": None if achieved is None else {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": "gemv_kernel: fused tier selection + tiered gather-GEMV "
                      "(fp16 full, int4 g128 approx)",
            "avg_launch_us": round(avg_us, 3),
            "launch_us": {"qkv": round(t_qkv * 1e6, 3), "o": round(t_o * 1e6, 3)},
            "bytes_per_launch": {"qkv": qkv_b, "o": o_b},
        },
        "kf": wl.kf, "ka": wl.ka,
        "mode": "graph" if graph is not None else "eager",
    }


def cpu_baseline(kf: int, ka: int, budget_s: float = 15.0):
    """The CPU oracle on a bounded sample of the same workload: weight set 0,
    tokens 0, 1, ... each ranking h and z and forming q, k, v and o, until
    about `budget_s` seconds of timed work are done."""
    import numpy as np

    import oracle as O
    import workloads as WL
    from workloads.accounting import gemv_algorithmic_bytes
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = 1
    mats = {}
    for m in ("q", "k", "v", "o"):
        Wt = WL.weights_fp16(CONFIG_ID, 0, m, HIDDEN, HIDDEN, 0.02)
        mats[m] = (O.ColumnStore("fp16", Wt), O.ColumnStore("int4", Wt))
    per_proj = gemv_algorithmic_bytes(HIDDEN, HIDDEN, kf, ka, "fp16", "int4")
    done, t_acc, tok = 0, 0.0, 0
    while t_acc < budget_s and tok < TOKENS:
        h = WL.laplace_fp16(CONFIG_ID, 0, "h", tok, HIDDEN)
        z = WL.laplace_fp16(CONFIG_ID, 0, "z", tok, HIDDEN)
        t0 = time.perf_counter()
        Fh, Ah = O.plan_tiers(h, kf, ka)
        for m in ("q", "k", "v"):
            O.tiered_gemv_fp16(h, Fh, Ah, *mats[m])
        Fz, Az = O.plan_tiers(z, kf, ka)
        O.tiered_gemv_fp16(z, Fz, Az, *mats["o"])
        t_acc += time.perf_counter() - t0
        done += 4
        tok += 1
    gbs = done * per_proj / t_acc / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{tok} tokens x (rank h, q, k, v; rank z, o) on weight set 0 "
                       f"({done} projections, {t_acc:.1f} s; numpy fp64)"),
            "us_per_projection": round(t_acc / done * 1e6, 1),
            "host_cores": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    r = gpu_run(args)
    base = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        base = cpu_baseline(r["kf"], r["ka"])
    gbs = r["step_bytes"] / r["sec_step"] / 1e9
    us_proj = r["sec_step"] / r["projections"] * 1e6
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["sec_step"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "us_per_projection": round(us_proj, 3),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "config": {
            "workload": ("7B-shaped attention projections q,k,v,o 4096x4096, fp16 W ~N(0,0.02) "
                         "column-major, int4 group-128 approx copy, skip/approx/full 40/30/30 %, "
                         "x ~Laplace(0,1) fp16, batch 1, 32 tokens per step over 32 weight sets"),
            "tokens_per_step": TOKENS,
            "weight_sets": args.sets,
            "k_full": r["kf"], "k_approx": r["ka"],
            "algorithmic_bytes_per_step": r["step_bytes"],
            "launch": r["mode"],
            "parallelism": "single GPU",
        },
        "roofline": r["roofline"],
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
