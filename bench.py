"""Benchmark of the three-tier activation-sparse decode path on one MI355X.

Headline workload (no --config): config 4, the 32-layer 7B projection
stream. Each layer has the seven projections of a 7B decoder layer in four
groups (q, k, v stacked 12288 x 4096 on h; o 4096 x 4096 on z; gate/up
interleaved 22016 x 4096 on x; down 4096 x 11008 on a = silu(g) * u), fp16
weights ~ N(0, 0.02) column-major with an int4 group-128 compressed copy,
tiers skip / approx / full = 50 / 25 / 25 % of each group's inputs, batch 1,
inputs ~ Laplace(0, 1) fp16. One step = 4 tokens x 32 layers = 128 layer
steps through spax_layer_step (one launch of the layer kernel each: every
group's ranking, tiered product and the SwiGLU epilogue). Layer l reads
weight set l (32 distinct sets, 13 GB), so weights come from HBM, not from
the 256 MB last-level cache.

The step is captured once in a HIP graph (through torch's graph capture on
the stream the library launches on) and replayed; warmup replays are
untimed, then exactly --steps replays are timed between two device
synchronisations. Inputs are resident in HBM before timing starts.

Printed: ONE JSON line with the throughput (effective weight GB/s on the
algorithmic bytes), microseconds per tiered projection, the roofline of the
layer kernel (its average launch duration from the timed replays, events
on the launch stream) and the CPU oracle timed on a bounded sample of the
same workload at one thread and at all host cores.

Other workloads (one JSON line each, same legs):
    --config 1   single 1024 x 1024 layer, 50/25/25 (no CPU leg)
    --config 2   7B-shaped attention projections q, k, v, o (4096 x 4096),
                 40/30/30, 32 tokens over 32 weight sets
    --config 3   7B SwiGLU FFN (gate/up 11008x4096, down 4096x11008), skip
                 30 / 50 / 70 %, approx 20 % (three lines, no CPU leg)
    --config 4 --host   weights in pinned host memory; only the selected
                 columns cross the host link
    --config 5   70B-shaped FFN, int4 full tier, int2 approx, 50/30/20

    --approx sign2   config 2 (or 1) with the SpAx page's two-scale 2-bit
                 sign code (section 5.1, Eq. 4) as the middle tier
    --approx trellis config 2 (or 1) with the trellis-coded middle tier
                 (section 5.1; GPU Viterbi encoder, 8 weight sets)
    --calibrate  the offline tier-size calibration of section 5.2 (steps 1 and
                 2) on the 7B attention groups, through the library

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--eager]
                    [--no-cpu-baseline] [--calib-copy] [--config N] [--host]
                    [--approx int4|sign2|trellis] [--select ...]
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

METRIC = ("µs per tiered projection & effective weight GB/s (% of HBM peak), "
          "batch-1 decode")
HBM_PEAK_GBS = 8000.0
# spax_layer.kernel of every layer step (SPAX_KERNEL_*; --select)
KERNEL = 0
PCIE5_X16_GBS = 64.0


# counter summaries per workload (FETCH_SIZE and WRITE_SIZE runs), valid while
# the sources of the kernel they measured are unchanged: the layer kernel, and
# the per-group product (gemv_kernel)
PMC_SUMMARY = {4: os.path.join(ROOT, "profiles", "layer_kernel_7b_stream_pmc.txt"),
               5: os.path.join(ROOT, "profiles", "layer_kernel_70b_ffn_pmc.txt"),
               2: os.path.join(ROOT, "profiles", "layer_kernel_7b_attention_pmc.txt")}
GEMV_PMC_SUMMARY = {5: os.path.join(ROOT, "profiles", "gemv_kernel_70b_ffn_pmc.txt"),
                    2: os.path.join(ROOT, "profiles", "gemv_kernel_7b_attention_pmc.txt")}
KERNEL_SOURCES = ("layer.hip", "layer_plan.h", "block_common.h", "spax_internal.h", "api.cpp")
GEMV_SOURCES = ("gemv.hip", "block_common.h", "stream_common.h", "spax_internal.h", "api.cpp")


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "activation_sparse_decode_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(config: int, layer: bool = True):
    """HBM bytes per launch of the layer kernel (layer) or of the per-group
    product from the committed counter summary of this workload (FETCH_SIZE
    and WRITE_SIZE, scaled by a plain copy's reading), or None when there is
    none or that kernel's sources changed since the counters were taken."""
    table, sources = (PMC_SUMMARY, KERNEL_SOURCES) if layer else (GEMV_PMC_SUMMARY, GEMV_SOURCES)
    try:
        text = open(table[config]).read()
    except (OSError, KeyError):
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:"):
            vals["traffic"] = float(line.split(":", 1)[1])
        elif line.startswith("kernel sources sha256"):
            vals["sha"] = line.rsplit(":", 1)[1].strip()
    if vals.get("sha") != kernel_source_hash(sources) or "traffic" not in vals:
        return None
    return int(vals["traffic"])


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- workloads

@dataclasses.dataclass
class Spec:
    """One benchmark workload: which groups a layer has, their shapes and
    formats, the tier split, how many distinct weight sets rotate, and how
    many (token, layer) layer-steps one step runs."""
    config: int
    name: str
    hidden: int
    inter: int                 # 0: no FFN groups
    attn: bool                 # q,k,v + o groups
    o_only: bool = False       # a single plain projection (the o slot)
    full_fmt: str = "fp16"
    approx_fmt: str = "int4"
    split: tuple = (50, 25, 25)    # skip / approx / full %
    std: float = 0.02
    sets: int = 32
    tokens: int = 32
    layers_per_token: int = 1  # distinct sets each token walks through
    host: bool = False

    def describe(self) -> str:
        s, a, f = self.split
        approx = {"int4": "int4 g128", "int2": "int2 g128", "sign2": "two-scale 2-bit sign",
                  "trellis": "trellis-coded 2-bit"}[self.approx_fmt]
        full = {"fp16": "fp16", "int4": "int4 g128"}[self.full_fmt]
        return (f"{self.name}: skip/approx/full {s}/{a}/{f} %, {full} full + "
                f"{approx} approx, W ~N(0,{self.std}) column-major, "
                f"x ~Laplace(0,1) fp16, batch 1, {self.tokens} tokens x "
                f"{self.layers_per_token} layer(s) per step over {self.sets} weight sets"
                + (", weights in pinned host memory" if self.host else ""))


def attention_spec(approx_fmt: str = "int4") -> Spec:
    return Spec(2, "7B-shaped attention projections q,k,v,o 4096x4096", 4096, 0, True,
                approx_fmt=approx_fmt, split=(40, 30, 30))


HEADLINE_CONFIG = 4


def specs_for(config: int, host: bool, approx: str = "int4"):
    if config == 1:
        if approx == "trellis":
            # the trellis encoder runs on the host (65536 candidates per weight):
            # two weight sets
            return [Spec(1, "single linear layer 1024x1024", 1024, 0, False, o_only=True,
                         approx_fmt="trellis", sets=2)]
        return [Spec(1, "single linear layer 1024x1024", 1024, 0, False, o_only=True,
                     approx_fmt=approx)]
    if config == 2:
        return [attention_spec(approx)]
    if config == 3:
        return [Spec(3, f"7B-shaped SwiGLU FFN gate/up 11008x4096, down 4096x11008", 4096, 11008,
                     False, split=(s, 20, 80 - s), sets=16) for s in (30, 50, 70)]
    if config == 4:
        if host:
            return [Spec(4, "32-layer 7B projection stream (4 attn + 3 FFN per layer)", 4096,
                         11008, True, sets=32, tokens=1, layers_per_token=32, host=True)]
        return [Spec(4, "32-layer 7B projection stream (4 attn + 3 FFN per layer)", 4096, 11008,
                     True, sets=32, tokens=4, layers_per_token=32)]
    if config == 5:
        return [Spec(5, "70B-shaped FFN gate/up 28672x8192, down 8192x28672", 8192, 28672, False,
                     full_fmt="int4", approx_fmt="int2", split=(50, 30, 20), std=0.015,
                     sets=8, tokens=16)]
    raise SystemExit(f"unknown --config {config}")


FMT = {"fp16": 1, "int4": 2, "int2": 3, "sign2": 4, "trellis": 5}


def group_shapes(spec: Spec) -> dict:
    """Stored (rows, cols) of each present group: QKV, O, GATE_UP, DOWN."""
    H, I = spec.hidden, spec.inter
    shapes = {}
    if spec.attn:
        shapes[0] = (3 * H, H)
    if spec.attn or spec.o_only:
        shapes[1] = (H, H)
    if I:
        shapes[2] = (2 * I, H)
        shapes[3] = (H, I)
    return shapes


def group_counts(spec: Spec, g: int):
    import workloads as WL
    n = spec.inter if g == 3 else spec.hidden
    return WL.tier_counts(n, WL.TierSplit(*spec.split))


def group_bytes(spec: Spec, g: int) -> int:
    """Bytes the method must move for group g of one layer step (selected
    columns, codes and scales, x, index lists, y) -- see
    workloads.accounting."""
    from workloads.accounting import gemv_algorithmic_bytes
    rows, cols = group_shapes(spec)[g]
    kf, ka = group_counts(spec, g)
    b = gemv_algorithmic_bytes(rows, cols, kf, ka, spec.full_fmt, spec.approx_fmt)
    if g == 2:          # gate/up writes a = silu(g) * u: half the stored rows
        b -= rows
    return b


def layer_bytes(spec: Spec) -> int:
    return sum(group_bytes(spec, g) for g in group_shapes(spec))


class Workload:
    """Device-resident (or pinned-host) weights, inputs, outputs and lists."""

    def __init__(self, spec: Spec):
        import torch

        import activation_sparse_decode_token_amd as spax
        import workloads as WL
        from activation_sparse_decode_token_amd.layouts import (build_matrix, glu_interleave,
                                                                stack_rows)

        self.spax, self.spec = spax, spec
        dev = torch.device("cuda:0")
        H, I = spec.hidden, spec.inter
        sk, ap, fu = spec.split
        split = WL.TierSplit(sk, ap, fu)
        res = spax.RES_HOST_PINNED if spec.host else spax.RES_DEVICE
        ff, af = FMT[spec.full_fmt], FMT[spec.approx_fmt]

        def gen(s, m, rows, cols):
            return WL.weights_fp16_torch(spec.config, s, m, rows, cols, spec.std, dev)

        # the trellis tier's shared codebook (seeded N(0, 1) draws, fp16)
        cb = (torch.from_numpy(WL.trellis_codebook(spec.config)).to(dev)
              if spec.approx_fmt == "trellis" else None)
        self.codebook = cb

        # tier counts per group: QKV, O, GATE_UP, DOWN
        kq = WL.tier_counts(H, split)
        kd = WL.tier_counts(I, split) if I else (0, 0)
        self.k = {0: kq, 1: kq, 2: kq, 3: kd}
        self.present = [spec.attn, spec.attn or spec.o_only, I > 0, I > 0]
        kf = [self.k[g][0] if self.present[g] else 0 for g in range(4)]
        ka = [self.k[g][1] if self.present[g] else 0 for g in range(4)]
        self.layers, self.single = [], {g: [] for g in range(4)}
        self.shapes = {}
        for s in range(spec.sets):
            mats = [None] * 4
            if spec.attn:
                q, k_, v = (gen(s, m, H, H) for m in ("q", "k", "v"))
                st = stack_rows([q, k_, v])
                del q, k_, v
                mats[0] = build_matrix(st, ff, af, residency=res, codebook=cb, seg_rows=H)
                del st
            if spec.attn or spec.o_only:
                o = gen(s, "o" if spec.attn else "w", H, H)
                mats[1] = build_matrix(o, ff, af, residency=res, codebook=cb)
                del o
            if I:
                g_, u_ = gen(s, "gate", I, H), gen(s, "up", I, H)
                gu = glu_interleave(g_, u_)
                del g_, u_
                mats[2] = build_matrix(gu, ff, af, layout=spax.LAYOUT_GLU_INTERLEAVED,
                                       residency=res)
                del gu
                d = gen(s, "down", H, I)
                mats[3] = build_matrix(d, ff, af, residency=res)
                del d
            torch.cuda.synchronize()
            self.layers.append(spax.Layer.make(mats, kf, ka, kernel=KERNEL))
            for g in range(4):
                if mats[g] is not None:
                    only = [None] * 4
                    only[g] = mats[g]
                    self.single[g].append(spax.Layer.make(only, kf, ka, kernel=KERNEL))
                    self.shapes[g] = (mats[g].rows, mats[g].cols)
            if s % 8 == 7 or s == spec.sets - 1:
                log(f"  {s + 1}/{spec.sets} weight sets built")
        f16, i32 = torch.float16, torch.int32
        # one input / output slot per (token, layer) layer-step
        self.slots = spec.tokens * spec.layers_per_token
        self.io = []
        for i in range(self.slots):
            t, l = divmod(i, spec.layers_per_token)
            vec = lambda nm: WL.laplace_fp16_torch(spec.config, l, nm, t, H, dev)
            F = [torch.empty(max(1, kf[g]), dtype=i32, device=dev) for g in range(4)]
            A = [torch.empty(max(1, ka[g]), dtype=i32, device=dev) for g in range(4)]
            kw = dict(full_idx=tuple(F), approx_idx=tuple(A))
            if spec.attn:
                kw.update(h=vec("h"), qkv=torch.empty(3 * H, dtype=f16, device=dev))
            if spec.attn or spec.o_only:
                kw.update(z=vec("z"), o=torch.empty(H, dtype=f16, device=dev))
            if I:
                kw.update(x=vec("x"), a=torch.empty(I, dtype=f16, device=dev),
                          down=torch.empty(H, dtype=f16, device=dev))
            self.io.append(spax.LayerIO.make(**kw))
        wsb = spax.layer_workspace_bytes(self.layers[0])
        self.ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
        self.ws_bytes = wsb
        self.copy = spax.copy_init(torch.cuda.Stream()) if spec.host else None
        torch.cuda.synchronize()

    def group_bytes(self, g: int) -> int:
        return group_bytes(self.spec, g)

    def layer_bytes(self) -> int:
        return layer_bytes(self.spec)

    def step_bytes(self) -> int:
        return self.slots * self.layer_bytes()

    def projections_per_layer(self) -> int:
        p = 0
        if self.spec.attn:
            p += 4
        elif self.spec.o_only:
            p += 1
        if self.spec.inter:
            p += 3
        return p

    def layer_of(self, i: int):
        t, l = divmod(i, self.spec.layers_per_token)
        return self.layers[(t * self.spec.layers_per_token + l) % self.spec.sets]

    def step(self, stream=None):
        """Enqueue one step: every (token, layer) slot runs the layer's groups
        (one layer-kernel launch per slot with device-resident weights)."""
        spax = self.spax
        for i in range(self.slots):
            spax.layer_step(self.layer_of(i), self.io[i], self.ws, self.ws_bytes,
                            compute_stream=stream, copy=self.copy)


def time_steps(wl: Workload, steps: int, warmup: int, eager: bool):
    """Warm up, then time exactly `steps` steps between synchronisations.
    Returns (seconds per step by events, seconds per step by wall clock,
    mode, stream)."""
    import torch
    stream = torch.cuda.Stream()
    graph = None
    with torch.cuda.stream(stream):
        wl.step(stream)                      # eager warm pass (also loads code objects)
        torch.cuda.synchronize()
        if not eager:
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
        for _ in range(warmup):
            run_once()
        torch.cuda.synchronize()
        log(f"warmup done ({warmup} steps, {'eager' if graph is None else 'graph'})")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(steps):
            run_once()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms_event = ev0.elapsed_time(ev1)
    log(f"timed {steps} steps: wall {wall * 1e3:.2f} ms, events {ms_event:.2f} ms")
    return ms_event * 1e-3 / steps, wall / steps, ("graph" if graph is not None else "eager"), stream


def host_link_peak_gbs() -> float:
    """Pinned host -> device copy rate of one large contiguous buffer."""
    import torch
    n = 1 << 30
    h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        d.copy_(h, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    return 3 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9


def _oracle_layer(spec: Spec, layer: int = 0):
    """The oracle's stores of one layer of the workload (weight set `layer`)
    and its tier counts per group."""
    import oracle as O
    import workloads as WL
    H, I = spec.hidden, spec.inter
    split = WL.TierSplit(*spec.split)
    mats = {}

    def add(name, rows, cols):
        Wt = WL.weights_fp16(spec.config, layer, name, rows, cols, spec.std)
        mats[name] = (O.ColumnStore(spec.full_fmt, Wt), O.ColumnStore(spec.approx_fmt, Wt))

    if spec.attn:
        for m in ("q", "k", "v", "o"):
            add(m, H, H)
    elif spec.o_only:
        Wt = WL.weights_fp16(spec.config, layer, "w", H, H, spec.std)
        mats["o"] = (O.ColumnStore(spec.full_fmt, Wt), O.ColumnStore(spec.approx_fmt, Wt))
    if I:
        add("gate", I, H)
        add("up", I, H)
        add("down", H, I)
    kq = WL.tier_counts(H, split)
    ks = {"qkv": kq, "o": kq, "ffn": kq, "down": WL.tier_counts(I, split) if I else (0, 0)}
    return mats, ks


def cpu_baseline(spec: Spec, layer_bytes: int, budget_s: float = 8.0, max_tokens: int = 32):
    """The CPU oracle (numpy fp64, test infrastructure) on a bounded sample
    of the workload: weight set 0, tokens 0, 1, ... each running every group
    of the layer (rank, tiered products, SwiGLU, rank a, down) until about
    `budget_s` seconds of timed work are done, once with the BLAS pool at one
    thread and once at all host cores."""
    import oracle as O
    import workloads as WL
    from threadpoolctl import threadpool_info, threadpool_limits
    t_build = time.perf_counter()
    mats, ks = _oracle_layer(spec)
    log(f"oracle stores built in {time.perf_counter() - t_build:.1f} s")
    H = spec.hidden

    def leg(threads):
        with threadpool_limits(limits=threads):
            used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
            done, t_acc = 0, 0.0
            while t_acc < budget_s and done < max_tokens:
                tok = done
                h = WL.laplace_fp16(spec.config, 0, "h", tok, H) if spec.attn else None
                z = (WL.laplace_fp16(spec.config, 0, "z", tok, H)
                     if spec.attn or spec.o_only else None)
                x = WL.laplace_fp16(spec.config, 0, "x", tok, H) if spec.inter else None
                t0 = time.perf_counter()
                O.layer_step(mats, ks, h=h, z=z, x=x)
                t_acc += time.perf_counter() - t0
                done += 1
        return {"value": round(done * layer_bytes / t_acc / 1e9, 4), "cores": int(used),
                "layer_steps": done, "seconds": round(t_acc, 2),
                "ms_per_layer_step": round(t_acc / done * 1e3, 1)}

    one = leg(1)
    log(f"oracle, 1 thread: {one['value']} GB/s ({one['ms_per_layer_step']} ms per layer step)")
    ncpu = os.cpu_count() or 1
    allc = leg(ncpu)
    log(f"oracle, {allc['cores']} threads: {allc['value']} GB/s")
    return {"value": allc["value"], "unit": "GB/s", "cores": allc["cores"], "kind": "oracle",
            "sample": (f"weight set 0 (one layer's groups), tokens 0..{allc['layer_steps'] - 1}:"
                       f" {allc['layer_steps']} layer steps in {allc['seconds']} s at "
                       f"{allc['cores']} threads; {one['layer_steps']} in {one['seconds']} s at "
                       "1 thread; numpy fp64, algorithmic bytes as on the GPU"),
            "one_thread": {"value": one["value"], "unit": "GB/s", "cores": 1,
                           "ms_per_layer_step": one["ms_per_layer_step"]},
            "all_cores": {"value": allc["value"], "unit": "GB/s", "cores": allc["cores"],
                          "ms_per_layer_step": allc["ms_per_layer_step"]},
            "cpu_model": cpu_model(), "nproc": ncpu}


def dtype_label(spec: Spec) -> str:
    name = {"fp16": "fp16", "int4": "int4 g128 codes", "int2": "int2 g128 codes",
            "sign2": "2-bit sign codes", "trellis": "2-bit trellis codes"}
    return (f"{name[spec.full_fmt]} full + {name[spec.approx_fmt]} approx weights, fp16 "
            "activations, fp32 accumulate, fp16 out")


def result_line(spec: Spec, wl: Workload, args, sec_step: float, mode: str, extra=None):
    step_b = wl.step_bytes()
    gbs = step_b / sec_step / 1e9
    n_proj = wl.slots * wl.projections_per_layer()
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(spec),
        "data": "synthetic",
        "us_per_projection": round(sec_step / n_proj * 1e6, 3),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "config": {
            "workload": spec.describe(),
            "tokens_per_step": spec.tokens,
            "layers_per_token": spec.layers_per_token,
            "weight_sets": spec.sets,
            "k_full_approx": {g: list(wl.k[g]) for g in range(4) if wl.present[g]},
            "algorithmic_bytes_per_step": step_b,
            "launch": mode,
            "parallelism": "single GPU",
        },
    }
    if extra:
        line.update(extra)
    return line


def layer_kernel_runs(wl: Workload) -> bool:
    """Whether spax_layer_step runs these layers as one layer-kernel launch."""
    if KERNEL != 0 or wl.spec.host:
        return False
    try:
        wl.spax.layer_schedule(wl.layers[0], 0)
        return True
    except wl.spax.SpaxError:
        return False


def roofline(spec: Spec, wl: Workload, sec_step: float, mode: str):
    """Roofline of the product kernel: algorithmic bytes per launch over its
    average launch duration (the timed replays' event time on the launch
    stream over the launches they hold). With the layer kernel a layer step
    is one launch; otherwise every group is one fused ranking + product
    launch (gemv_kernel)."""
    if mode != "graph":
        return None
    layer = layer_kernel_runs(wl)
    per_slot = 1 if layer else len(group_shapes(spec))
    launches = wl.slots * per_slot
    t_launch = sec_step / launches
    bytes_launch = wl.layer_bytes() / per_slot
    achieved = bytes_launch / t_launch / 1e9
    log(f"{'layer' if layer else 'product'} kernel: {t_launch * 1e6:.2f} us per launch, "
        f"{achieved:.0f} GB/s on algorithmic bytes")
    return {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": (measured_traffic(spec.config, layer)
                    if spec.approx_fmt in ("int4", "int2") else None),
        "kernel": ("layer_kernel: every group of one decoder layer (ranking, tiered "
                   "gather-GEMV, SwiGLU) in one launch" if layer else
                   "gemv_kernel: fused tier selection + tiered gather-GEMV, one launch per "
                   "group (the mean over the groups' launches)"),
        "avg_launch_us": round(t_launch * 1e6, 3),
        "launches_per_step": launches,
        "bytes_per_launch": int(bytes_launch),
    }


def run_spec(spec: Spec, args, cpu_leg: bool):
    import torch
    log(f"config {spec.config}: {spec.describe()}")
    t0 = time.perf_counter()
    wl = Workload(spec)
    log(f"weights ready in {time.perf_counter() - t0:.1f} s")
    eager = args.eager or spec.host
    sec_step, _, mode, _ = time_steps(wl, args.steps, args.warmup, eager)
    extra = {"roofline": roofline(spec, wl, sec_step, mode)}
    if spec.host:
        peak = host_link_peak_gbs()
        link = wl.step_bytes() / sec_step / 1e9
        extra["host_link"] = {
            "achieved": round(link, 2), "unit": "GB/s",
            "copy_peak_measured": round(peak, 2), "nominal_pcie5_x16": PCIE5_X16_GBS,
            "frac_of_measured_peak": round(link / peak, 4),
            "note": "selected columns and scales copied from pinned host memory each "
                    "step, overlapped with the product; bytes = algorithmic bytes",
        }
        log(f"host link: {link:.1f} GB/s effective, plain pinned copy {peak:.1f} GB/s")
    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy: 268435456 bytes read, 268435456 bytes written")
    layer_b = wl.layer_bytes()
    line = result_line(spec, wl, args, sec_step, mode, extra)
    del wl
    torch.cuda.empty_cache()
    base = None
    if cpu_leg and not args.no_cpu_baseline and spec.approx_fmt != "trellis":
        # (the trellis oracle's numpy Viterbi needs seconds per column, so
        # that line has no CPU leg)
        log("timing the CPU oracle on a bounded sample")
        base = cpu_baseline(spec, layer_b, max_tokens=2 if spec.config == 5 else 32)
    line["cpu_baseline"] = base
    return line


def run_main(args):
    import torch

    import activation_sparse_decode_token_amd as spax
    spax.lib()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (torch.cuda.is_available() is False)")
    log(f"device {torch.cuda.get_device_name(0)}")
    config = HEADLINE_CONFIG if args.config is None else args.config
    specs = specs_for(config, args.host, args.approx)
    for spec in specs:
        if config == 2:
            spec.sets = args.sets
            if spec.approx_fmt == "trellis":
                # the offline Viterbi encoding takes about a second per weight
                # set (16 GB of backpointers per launch): 8 sets, still far
                # past the 256 MB last-level cache
                import activation_sparse_decode_token_amd.layouts as LY
                LY.TRELLIS_WS_BYTES = 16 << 30
                spec.sets = min(args.sets, 8)
        line = run_spec(spec, args, cpu_leg=config in (2, 4, 5) and not spec.host)
        print(json.dumps(line), flush=True)


def run_calibrate(args):
    """Offline tier-size calibration (SpAx page section 5.2) on the 7B
    attention groups: Step 1 to a 40 % layer budget, then Step 2's grid at
    each group's budget, every evaluation through the library's kernels.
    One JSON line: evaluations per second (one evaluation = one grid
    setting over the calibration tokens, each token one ranking plus one
    tiered product, against dense references taken once)."""
    import torch

    import activation_sparse_decode_token_amd as spax
    import activation_sparse_decode_token_amd.calibrate as K
    import workloads as WL
    from activation_sparse_decode_token_amd.layouts import build_matrix, stack_rows
    spax.lib()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (torch.cuda.is_available() is False)")
    dev = torch.device("cuda:0")
    H, tokens, steps, target = 4096, 8, 10, 40
    gen = lambda m: WL.weights_fp16_torch(2, 0, m, H, H, 0.02, dev)
    qkv = build_matrix(stack_rows([gen("q"), gen("k"), gen("v")]))
    o = build_matrix(gen("o"))
    vec = lambda nm, t: WL.laplace_fp16_torch(2, 0, nm, t, H, dev)
    t0 = time.perf_counter()
    groups = [K.Group(qkv, [vec("h", t) for t in range(tokens)]),
              K.Group(o, [vec("z", t) for t in range(tokens)])]
    budgets, rounds = K.step1(groups, target)
    chosen = [K.step2(g, b, steps) for g, b in zip(groups, budgets)]
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    evals = sum(g.evaluations for g in groups)   # one per budget or grid setting tried
    line = {
        "metric": "offline tier-size calibration (SpAx page section 5.2, steps 1 and 2): "
                  "evaluations per second",
        "value": round(evals / sec, 2), "unit": "evaluations/s", "n_gpus": 1,
        "higher_is_better": True, "data": "synthetic", "dtype": "fp32",
        "seconds": round(sec, 3), "evaluations": evals,
        "config": {"workload": "7B-shaped attention groups (q,k,v stacked 12288x4096; o "
                               "4096x4096), fp16 full + int4 g128 approx, W ~N(0,0.02), "
                               f"{tokens} calibration tokens of Laplace(0,1) inputs per group, "
                               f"layer budget target {target} %, step-2 grid of {steps} steps",
                   "tokens": tokens},
        "step1_budgets_pct": {"qkv": budgets[0], "o": budgets[1]},
        "step1_rounds": len(rounds),
        "step2_choice": {"qkv": list(chosen[0][0]), "o": list(chosen[1][0])},
        "step2_tables": {"qkv": [list(r[:2]) + [r[2]] for r in chosen[0][1]],
                         "o": [list(r[:2]) + [r[2]] for r in chosen[1][1]]},
    }
    if not args.no_cpu_baseline:
        import oracle as O
        import oracle.spax_calibrate as C
        Wt = WL.weights_fp16(2, 0, "o", H, H, 0.02)
        mats = [(O.ColumnStore("fp16", Wt), O.ColumnStore("int4", Wt))]
        xs = [WL.laplace_fp16(2, 0, "z", t, H) for t in range(tokens)]
        kt, km = chosen[1][0]
        c0 = time.perf_counter()
        C.group_error(mats, xs, kt, km)
        csec = time.perf_counter() - c0
        line["cpu_baseline"] = {"value": round(1.0 / csec, 4), "unit": "evaluations/s",
                                "kind": "oracle", "cores": os.cpu_count(),
                                "sample": f"one evaluation of the o group ({tokens} tokens, "
                                          f"k_top={kt}, k_mid={km}; numpy fp64)"}
    print(json.dumps(line), flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--sets", type=int, default=32,
                   help="distinct weight sets rotated over the tokens (config 2; default 32)")
    p.add_argument("--eager", action="store_true",
                   help="launch every kernel from Python instead of replaying a graph")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one plain 256 MiB device copy (counter calibration)")
    p.add_argument("--config", type=int, default=None,
                   help="benchmark workload (1-5; default 4, the 32-layer 7B stream)")
    p.add_argument("--host", action="store_true",
                   help="with --config 4: weights in pinned host memory")
    p.add_argument("--approx", choices=("int4", "sign2", "trellis"), default="int4",
                   help="middle tier of config 2 or config 1: int4 "
                        "group-128 (default), the two-scale 2-bit sign code or the trellis code")
    p.add_argument("--calibrate", action="store_true",
                   help="run the offline tier-size calibration (steps 1 and 2) on the 7B "
                        "attention groups instead of the decode benchmark")
    p.add_argument("--select", choices=("fused", "layer", "per_group", "separate"),
                   default="fused",
                   help="launch form of each layer step: the one-launch layer kernel "
                        "(fused, the default), one fused launch per group, or a separate "
                        "selection kernel per group")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    if args.select != "fused":
        global KERNEL
        KERNEL = {"layer": 0, "separate": 1, "per_group": 2}[args.select]
    if args.calibrate:
        run_calibrate(args)
        return
    run_main(args)


if __name__ == "__main__":
    main()
