#!/usr/bin/env python3
"""Benchmark of the DFlash drafter block step on one MI355X.

One step = one block step (embed, 5 drafter layers with ring + block
attention, output norm, lm_head, greedy drafts) plus the device-side
acceptance scan, on inputs already resident in HBM: by default a replay of
the step captured in a HIP graph (one graph per step of the sequence, each
reading that step's inputs where they lie); --launch eager launches it
directly on the stream instead (dflash_block_step_accept, about 6 us faster
per step), and every line also reports the other launch mode's time on the
same steps. Default workload: real
drafter dimensions (5 layers, n_embd 6656, heads 32/8, head_dim 128, n_ff
19968, window 2048, block 16, vocab 8192), bf16 weights and bf16 ring, ring full
(positions 0..2047 injected), n_past 2048; every step gets a fresh id_last and a
target that copies that step's drafts up to a planted mismatch index (learned
in an untimed pass over the same step sequence).

Prints one JSON line: value = achieved HBM GB/s of the whole step (algorithmic
bytes / step time), with the step time in ms_per_step and step_us, a roofline
object for the dominant kernel (the gate/up GEMV) and the CPU oracle's rate
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "drafter block-step µs + achieved HBM GB/s (% of peak), real dims bf16, 1 MI355X"
HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "gate_up_gemv_counters.json")
KERNEL_SRC = [os.path.join(ROOT, "block_diffusion_drafter_02_amd", "csrc", f)
              for f in ("kernels_weights.hip", "gemv_device.h", "dflash_internal.h")]

WORKLOADS = {
    # name: (weight dtype, ring dtype, feature dtype, batch, positions injected before every step, block width,
    #        draft sampling temperature)
    "bf16": ("bf16", "bf16", "bf16", 1, 0, 16, 0.0),
    "f32": ("f32", "f32", "f32", 1, 0, 16, 0.0),
    "bf16-batch8": ("bf16", "bf16", "bf16", 8, 0, 16, 0.0),
    "fp8-inject512": ("fp8", "bf16", "bf16", 1, 512, 16, 0.0),
    "bf16-g4": ("bf16", "bf16", "bf16", 1, 0, 4, 0.0),
    "bf16-sample": ("bf16", "bf16", "bf16", 1, 0, 16, 1.0),
    "bf16-paged": ("bf16", "bf16", "bf16", 1, 0, 16, 0.0),
}
PAGED = {"bf16-paged"}  # rings live in 128-slot pages of one pool, named by shuffled block tables
FEATURE_POOL = 4  # distinct resident feature blocks cycled by the per-step inject (content does not change cost)


def esize(dt: str) -> float:
    return {"f32": 4, "bf16": 2, "fp8": 1}[dt]


def step_bytes(shape, wdt: str, rdt: str, n_vis: list[int]) -> dict:
    """Algorithmic HBM bytes of one block step: every streamed weight once (plus fp8 row scales), the visible
    ring K/V of every layer once per sequence, the norm vectors, the embedding rows, the logits."""
    E, F, V, L = shape.n_embd, shape.n_ff, shape.n_vocab, shape.n_layer
    qdim, kvdim = shape.q_dim, shape.kv_dim
    per_layer = (qdim + 2 * kvdim) * E + E * qdim + 2 * F * E + E * F
    w = (L * per_layer + V * E) * esize(wdt)
    if wdt == "fp8":
        w += (L * (qdim + 2 * kvdim + E + 2 * F + E) + V) * 4
    aux = "f32" if wdt == "f32" else "bf16"
    B = len(n_vis)
    ring = sum(L * shape.n_head_kv * nv * shape.head_dim * 2 * esize(rdt) for nv in n_vis)
    norms = (L * (2 * E + 2 * shape.head_dim) + E) * 4
    embed = 16 * B * E * esize(aux)
    logits = 16 * B * V * 4 + B * 15 * 4
    return {"weights": w, "ring": ring, "other": norms + embed + logits, "total": w + ring + norms + embed + logits}


def inject_bytes(shape, T: int, wdt: str, rdt: str, fdt: str) -> dict:
    """Algorithmic HBM bytes of encoding and injecting T positions: the features and fc once, the fused
    wk/wv of all layers once (plus fp8 row scales), h [T, n_embd] f32 written once and read once, the ring
    K/V entries and slot table written."""
    E, L, C = shape.n_embd, shape.n_layer, shape.n_capture * shape.target_hidden
    aux = "f32" if wdt == "f32" else "bf16"
    kvrows = L * 2 * shape.kv_dim
    w = C * E * esize(aux) + kvrows * E * esize(wdt) + (kvrows * 4 if wdt == "fp8" else 0)
    io = T * C * esize(fdt) + 2 * T * E * 4 + T * 4
    ring = T * kvrows * esize(rdt) + T * 4
    flops_enc = 2.0 * T * C * E
    flops_kv = 2.0 * T * E * kvrows
    return {"weights": w, "io": io, "ring": ring, "total": w + io + ring, "flops_encode": flops_enc,
            "flops_kv": flops_kv}


def visible_slots(n_past: int, window: int, block: int) -> int:
    """Ring slots visible to at least one block row when positions 0..n_past-1 were injected in order."""
    lo = max(0, n_past - window)  # oldest position still held by the ring
    # row 0 (position n_past) sees positions > n_past - window
    return n_past - max(lo, n_past - window + 1)


def kernel_src_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(bytes_per_launch_alg: float):
    """HBM bytes per launch of the gate/up GEMV from committed rocprofv3 counter runs, or None when the kernel
    source changed since they were taken."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    if c.get("kernel_src_sha256_16") != kernel_src_hash():
        return None
    return c.get("hbm_bytes_per_launch")


GU_KERNEL = "gemv_kernel<1, 1, 1, 2, 1, 4, 64>"  # bf16 weights, f32 activations split at load, one row tile, SwiGLU, 4 waves, 64 columns
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_means(run_dir: str, counter: str) -> tuple[float, float]:
    """(mean per dispatch of the gate/up GEMV, mean of the five largest device copies) of one rocprofv3 --pmc
    counter in KiB, from the counter_collection CSV under run_dir."""
    import csv
    import glob

    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    gu, copies = [], []
    for f in files:
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            v = float(r["Counter_Value"])
            if GU_KERNEL in r["Kernel_Name"]:
                gu.append(v)
            elif COPY_KERNEL in r["Kernel_Name"]:
                copies.append(v)
    if not gu or len(copies) < 5:
        raise SystemExit(f"{counter}: {len(gu)} gate/up dispatches, {len(copies)} copies in {run_dir}")
    top = sorted(copies)[-5:]
    return sum(gu) / len(gu), sum(top) / len(top)


def write_counters(fetch_dir: str, write_dir: str, copy_mib: int, commands: list[str]) -> dict:
    """Reduce two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, each with a device copy of copy_mib MiB
    for calibration) to the HBM bytes per gate/up launch, stored with the hash of the kernel sources."""
    fetch, fcopy = _counter_means(fetch_dir, "FETCH_SIZE")
    write, wcopy = _counter_means(write_dir, "WRITE_SIZE")
    n = copy_mib << 20
    ff, wf = n / (fcopy * 1024.0), n / (wcopy * 1024.0)  # true bytes per counted byte, from a copy of known size
    from block_diffusion_drafter_02_amd import synth

    sh = synth.REAL
    alg = 2 * sh.n_ff * sh.n_embd * 2 + 16 * (sh.n_embd + sh.n_ff) * 4
    out = {
        "kernel": f"void {GU_KERNEL}(GemvArgs)",
        "workload": "real-dimension bf16 block step, gate/up projection + SwiGLU (one launch per layer)",
        "fetch_size_kib_per_dispatch": round(fetch, 1),
        "write_size_kib_per_dispatch": round(write, 1),
        "calibration": {"kernel": COPY_KERNEL, "bytes": n, "fetch_size_kib": round(fcopy, 3),
                        "write_size_kib": round(wcopy, 3), "fetch_factor": round(ff, 4),
                        "write_factor": round(wf, 4)},
        "hbm_bytes_per_launch": int(round(fetch * 1024.0 * ff + write * 1024.0 * wf)),
        "algorithmic_bytes_per_launch": alg,
        "kernel_src_sha256_16": kernel_src_hash(),
        "commands": commands,
        "kernel_src": [os.path.relpath(f, ROOT) for f in KERNEL_SRC],
    }
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
    return out


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's processor string."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(shape, raw, wdt, rdt, n_past, total_bytes, inject_feats=None, runs=3, block_width=16):
    """The oracle, as it stands, for block steps of one sequence at the same dimensions on a synthetic ring
    with the same fill (each preceded by encoding and injecting ``inject_feats`` when given): the median of
    ``runs`` steps with the BLAS thread pool as configured, then one step on a single thread. Returns the
    rates in the metric's unit (algorithmic GB/s)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import dflash_oracle as O

    cfg = dataclasses.replace(O.Config.from_shape(shape, rdt), block=block_width)
    w = O.Weights(raw, wdt)
    ring = O.Ring(cfg)
    rng = np.random.default_rng(0)
    rnd = O.round_bf16 if rdt == "bf16" else O.round_f32
    ring.K[:] = rnd(rng.standard_normal(ring.K.shape))
    ring.V[:] = rnd(rng.standard_normal(ring.V.shape))
    held = np.arange(max(0, n_past - cfg.window), n_past)
    ring.slot_pos[held % cfg.window] = held
    ring.written[held % cfg.window] = True
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    if wdt == "fp8":
        # the GPU quantises at setup, outside its clock; so does the oracle here
        for l in range(cfg.n_layer):
            for name in O.Weights.MATS:
                w.fp8_codes((l, name))
        w.fp8_codes("lm_head")
    state = {"np": n_past, "k": 0}

    def one_step() -> float:
        t0 = time.perf_counter()
        if inject_feats is not None:
            T = inject_feats.shape[0]
            O.inject(cfg, w, ring, O.encode(cfg, w, inject_feats), np.arange(state["np"], state["np"] + T))
            state["np"] += T
        O.block_forward(cfg, w, ring, O.block_ids(cfg, 1 + state["k"]), state["np"])
        state["k"] += 1
        return time.perf_counter() - t0

    per = [one_step() for _ in range(runs)]
    med = float(np.median(per))
    with threadpool_limits(limits=1):
        single = one_step()
    inj = f", each after injecting {inject_feats.shape[0]} positions" if inject_feats is not None else ""
    return {"value": round(total_bytes / med / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "seconds_per_step_median": round(med, 3),
            "seconds_per_step": [round(t, 3) for t in per],
            "single_thread": {"value": round(total_bytes / single / 1e9, 4), "seconds_per_step": round(single, 3)},
            "sample": f"{runs} block steps of one sequence (5 layers + lm_head, block width {cfg.block}) at the same "
                      f"dimensions and dtypes{inj}, ring filled to n_past={n_past} with synthetic values (content does "
                      f"not change the cost), median taken, then one more step on one thread; the rate is this "
                      f"workload's algorithmic bytes per step over the oracle's time per step"}


# Figures the dflash-ops card (Measured) reports for its own build on an RTX 6000 Ada (sm89): context for
# this GPU's numbers, not a target on the same machine.
PAGE_CONTEXT = {
    "source": "dflash-ops card, Measured (RTX 6000 Ada, real dims, ring 2048, vocab 8192)",
    "gemm_weight_stream_gbs": [720, 736],
    "read_bandwidth_gbs": 771,
    "non_gemm_share": {"fp32_weights": 0.18, "bf16_weights": 0.30},
}

# Kernels of a block step that stream no weights (the rest are the weight-streaming projections).
NON_GEMM = ("attn_partial_kernel", "attn_combine_kernel", "embed_kernel", "accept_kernel")
STEP_FIRST = ("embed_kernel", "chain_head_kernel")  # the first kernel of every block step


def summarize_trace(run_dir: str, skip_steps: int = 5) -> dict:
    """Per-kernel durations, per-step span (first kernel start to last kernel end of one block step) and
    the non-GEMM share of kernel time from a rocprofv3 --kernel-trace CSV of bench runs. Steps are cut at
    the first kernel of each step; setup kernels before the first step and after the last are dropped, and
    so are the first ``skip_steps`` steps."""
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in csv.DictReader(open(f))]
    rows.sort()
    starts = [i for i, r in enumerate(rows) if r[2].startswith(STEP_FIRST)]
    if len(starts) < skip_steps + 2:
        raise SystemExit(f"{run_dir}: {len(starts)} block steps in the trace")
    spans, per_kernel, gemm_t, other_t = [], {}, 0.0, 0.0
    for a, b in zip(starts[skip_steps:-1], starts[skip_steps + 1:]):
        step = [r for r in rows[a:b] if not r[2].startswith("__amd_rocclr")]
        # a step ends with the projection that writes the logits; later kernels belong to the host loop
        spans.append((max(r[1] for r in step) - step[0][0]) / 1e3)
        for t0, t1, name in step:
            short = name.split("(")[0].replace("void ", "")
            per_kernel.setdefault(short, []).append((t1 - t0) / 1e3)
            if short.startswith(NON_GEMM):
                other_t += (t1 - t0) / 1e3
            else:
                gemm_t += (t1 - t0) / 1e3
    n = len(spans)
    kern = {k: {"calls_per_step": round(len(v) / n, 2), "median_us": round(float(np.median(v)), 2),
                "us_per_step": round(sum(v) / n, 2)} for k, v in sorted(per_kernel.items(), key=lambda kv: -sum(kv[1]))}
    return {"steps": n, "span_us_median": round(float(np.median(spans)), 2),
            "span_us_p10": round(float(np.percentile(spans, 10)), 2),
            "span_us_p90": round(float(np.percentile(spans, 90)), 2),
            "kernel_us_per_step": round((gemm_t + other_t) / n, 2),
            "non_gemm_share": round(other_t / (gemm_t + other_t), 4), "kernels": kern}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=50)
    ap.add_argument("--path", default="auto", choices=["auto", "kernels", "persistent"],
                    help="block-step path (auto: the per-launch kernels; persistent: the opt-in persistent chain)")
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="how each timed step is launched: graph (a replay of the step captured with "
                         "dflash_step_graph_create, the default) or eager (dflash_block_step_accept on the stream)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (five times) to calibrate byte counters")
    ap.add_argument("--summarize-trace", metavar="RUN_DIR",
                    help="summarise a rocprofv3 --kernel-trace run of this bench (per-kernel times, per-step span, "
                         "non-GEMM share) as JSON, then exit (no GPU needed)")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="reduce two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of a --calibrate-copy-mib bench "
                         "into the committed gate/up traffic figures, then exit (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace)), flush=True)
        return 0
    if args.write_counters:
        mib = args.calibrate_copy_mib or 1024
        cmd = ("rocprofv3 --pmc {c} -d {d} -o run --output-format csv -- python3 -u bench.py --steps 3 --warmup 1 "
               f"--no-cpu-baseline --stage-reps 3 --calibrate-copy-mib {mib}")
        out = write_counters(args.write_counters[0], args.write_counters[1], mib,
                             [cmd.format(c="FETCH_SIZE", d=args.write_counters[0]),
                              cmd.format(c="WRITE_SIZE", d=args.write_counters[1])])
        print(json.dumps(out), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the drafter library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import torch

    from block_diffusion_drafter_02_amd import _lib, synth
    from block_diffusion_drafter_02_amd.drafter import Drafter, to_device

    wdt, rdt, fdt, B, T_inj, g, temp = WORKLOADS[args.workload]
    shape = synth.REAL
    t_setup = time.perf_counter()
    print(f"[bench] generating {args.workload} weights", file=sys.stderr, flush=True)
    raw = synth.weights(shape, wdt, seed=0)
    if B == 1:
        n_pasts = [2300] if wdt == "f32" else [2048]
    else:
        n_pasts = [int(v) for v in synth.batch_n_past(B, seed=0)]
    dr = Drafter(shape, raw, wdt, rdt, fdt, max_batch=B, max_inject=shape.window)
    dr.set_path({"auto": _lib.PATH_AUTO, "kernels": _lib.PATH_KERNELS, "persistent": _lib.PATH_PERSISTENT}[args.path])
    print("[bench] injecting context", file=sys.stderr, flush=True)
    rings = []
    paged = args.workload in PAGED
    if paged:
        n_tab = shape.window // dr.PAGE_SLOTS
        pool = dr.new_pool(n_tab * B)
        page_ids = np.random.default_rng(0).permutation(n_tab * B).astype(np.int32)
    for b in range(B):
        rings.append(torch.from_numpy(page_ids[b * n_tab:(b + 1) * n_tab]).to(dr.device) if paged else dr.new_ring())

    def fill_rings():
        """Reset every ring and inject its context: the last window of positions before n_past (f32: from
        the start of the window before, so the ring wraps)."""
        if paged:
            dr.pages_reset(0, n_tab * B)
        for b, n in enumerate(n_pasts):
            if not paged:
                dr.ring_reset(rings[b])
            first = max(0, n - (n // shape.window + 1) * shape.window) if wdt == "f32" else max(0, n - shape.window)
            pos = np.arange(first, n, dtype=np.int32)
            feats = to_device(synth.features(shape, len(pos), fdt, seed=0, tag=f"bench.feats{b}"), dr.device)
            for c0 in range(0, len(pos), shape.window):
                sl = slice(c0, c0 + shape.window)
                h = dr.encode(feats[sl])
                dr.inject(rings[b], h, torch.from_numpy(pos[sl]).to(dr.device))
            del feats
        torch.cuda.synchronize()

    fill_rings()
    table = dr.ring_table(rings)
    n_vis = [visible_slots(n, shape.window, shape.block) for n in n_pasts]
    nb = step_bytes(shape, wdt, rdt, n_vis)
    K, W = args.steps, args.warmup
    ib = None
    if T_inj:
        # every step first injects T_inj new positions [n_past, n_past + T_inj), then steps at the new n_past
        ib = inject_bytes(shape, T_inj, wdt, rdt, fdt)
        pool = [to_device(synth.features(shape, T_inj, fdt, seed=0, tag=f"bench.inject{i}"), dr.device)
                for i in range(FEATURE_POOL)]
        h_inj = torch.empty((T_inj, shape.n_embd), dtype=torch.float32, device=dr.device)
        starts = n_pasts[0] + T_inj * np.arange(W + K + 1, dtype=np.int64)
        pos_all = torch.from_numpy((starts[:, None] + np.arange(T_inj)[None]).astype(np.int32)).to(dr.device)
        np_all = torch.from_numpy((starts[1:, None]).astype(np.int32)).to(dr.device)
    ids_all = torch.from_numpy(synth.integers(0, "bench.id_last", (W + K, B), 0, shape.n_vocab)).to(dr.device)
    dr.set_block_width(g)
    dr.set_sampling(temp, 0x5EED)
    # per step and sequence: a fresh id_last and a planted mismatch index m ~ U{0..g-1} (m = g-1: none); the
    # target copies that step's drafts before m, differs at m, and is uniform filler after it
    mism_all = synth.integers(0, "bench.mismatch", (W + K, B), 0, g)
    fill_all = synth.integers(0, "bench.target", (W + K, B, g - 1), 0, shape.n_vocab)
    tgt_all = torch.from_numpy(fill_all).to(dr.device)
    # per-step inputs side by side ([id_last (B) | target (B x (g-1))]); `inputs` is the fixed buffer of the
    # one graph that times replays alone
    inputs_all = torch.cat([ids_all, tgt_all.reshape(W + K, B * (g - 1))], dim=1).contiguous()
    inputs = inputs_all[0].clone()
    il = inputs[:B]
    target = inputs[B:].view(B, g - 1)
    npst = torch.tensor(n_pasts, dtype=torch.int32, device=dr.device)
    logits = torch.empty((16 * B, shape.n_vocab), dtype=torch.float32, device=dr.device)
    drafts = torch.empty((B, g - 1), dtype=torch.int32, device=dr.device)
    n_ok = torch.empty((B,), dtype=torch.int32, device=dr.device)
    stream = torch.cuda.Stream()
    graph = dr.capture_step(table, il, npst, logits, drafts, target, n_ok, stream=stream)
    # one captured step per step of the sequence, reading that step's row of the resident input table (and
    # n_past) where it lies, as a verifier that writes its outputs into a graph's input buffers would leave
    # them: no per-step refresh copy
    print("[bench] capturing one graph per step", file=sys.stderr, flush=True)
    step_graphs = [dr.capture_step(table, inputs_all[k][:B], np_all[k] if T_inj else npst, logits, drafts,
                                   inputs_all[k][B:].view(B, g - 1), n_ok, stream=stream) for k in range(W + K)]

    def inject_step(k):
        dr.encode(pool[k % FEATURE_POOL], h_inj, stream=stream)
        dr.inject(rings[0], h_inj, pos_all[k], stream=stream)

    def step(k, mode=None):
        if T_inj:
            inject_step(k)
        if (mode or args.launch) == "graph":  # the step's own graph, over its row of the input table
            step_graphs[k].launch(stream)
        else:  # an eager step takes this step's inputs where they lie
            row = inputs_all[k]
            dr.block_step(table, row[:B], np_all[k] if T_inj else npst, out=(logits, drafts), stream=stream,
                          target=row[B:].view(B, g - 1), n_ok=n_ok)

    # untimed pass over the same step sequence: learn each step's drafts and plant its target
    print("[bench] planting per-step targets", file=sys.stderr, flush=True)
    with torch.cuda.stream(stream):
        for k in range(W + K):
            step(k)
            stream.synchronize()
            planted = synth.planted_targets(drafts.cpu().numpy(), mism_all[k], fill_all[k], shape.n_vocab)
            inputs_all[k, B:] = torch.from_numpy(planted.reshape(-1)).to(dr.device)
    if T_inj:  # the injections advanced the context: start again from the same state
        fill_rings()
        npst.copy_(torch.tensor(n_pasts, dtype=torch.int32))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    with torch.cuda.stream(stream):
        for k in range(W):
            step(k)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for k in range(K):
            step(W + k)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ev_ms = e0.elapsed_time(e1) / K
        n_ok_last = n_ok.cpu().numpy()
        accept_ok = bool(np.array_equal(n_ok_last, mism_all[W + K - 1]))
        # per-step spread: the same K steps again, an event recorded before each (outside the timed pass: the
        # events themselves add about 5 us per step)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        for k in range(K):
            ev[k].record(stream)
            step(W + k)
        ev[K].record(stream)
        torch.cuda.synchronize()
        per_step_us = np.array([ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(K)])
        # the same K steps launched the other way
        other = "eager" if args.launch == "graph" else "graph"
        o0, o1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        o0.record(stream)
        for k in range(K):
            step(W + k, other)
        o1.record(stream)
        torch.cuda.synchronize()
        other_ms = o0.elapsed_time(o1) / K
        # steps alone, without the per-step input refresh: graph replays, then eager launches
        g0, g1, g2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        g0.record(stream)
        for k in range(K):
            graph.launch(stream)
        g1.record(stream)
        for k in range(K):
            dr.block_step(table, il, npst, out=(logits, drafts), stream=stream, target=target, n_ok=n_ok)
        g2.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / K
        eager_ms = g1.elapsed_time(g2) / K
        # dominant kernel of the block step: the gate/up GEMV of layer 0, launched alone on the same stream
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            dr.replay_stage(_lib.STAGE_GATE_UP, 0, stream)
        r0.record(stream)
        for _ in range(args.stage_reps):
            dr.replay_stage(_lib.STAGE_GATE_UP, 0, stream)
        r1.record(stream)
        torch.cuda.synchronize()
        gu_ms = r0.elapsed_time(r1) / args.stage_reps
        inj = None
        if T_inj:
            # the per-step injection alone (encode GEMM + norm, then the fused wk/wv GEMM + ring writes) and
            # the encode alone, on the same stream; the ring is re-filled at positions already written
            reps = max(5, min(args.stage_reps, 20))
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            for k in range(reps):
                inject_step(W + K - 1 - (k % 4))
            e[1].record(stream)
            for k in range(reps):
                dr.encode(pool[k % FEATURE_POOL], h_inj, stream=stream)
            e[2].record(stream)
            torch.cuda.synchronize()
            inj = {"inject_us": e[0].elapsed_time(e[1]) / reps * 1e3, "encode_us": e[1].elapsed_time(e[2]) / reps * 1e3}
    if args.path == "persistent" or dr.step_path(B) == _lib.PATH_PERSISTENT:
        dr.check_device(stream)  # raises if a bounded wait of the chain gave up during the run

    ms = wall * 1e3 / K
    total = nb["total"] + (ib["total"] if ib else 0)
    value = total / (ms * 1e-3) / 1e9
    E, F = shape.n_embd, shape.n_ff
    gu_bytes = 2 * F * E * esize(wdt) + 16 * B * E * 4 + 16 * B * F * 4
    if wdt == "fp8":
        gu_bytes += 2 * F * 4
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    traffic = read_traffic(gu_bytes)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "step_us": round(ms * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "event_ms_per_step": round(ev_ms, 5),
        "step_us_median": round(float(np.median(per_step_us)), 2),
        "step_us_p10": round(float(np.percentile(per_step_us, 10)), 2),
        "step_us_p90": round(float(np.percentile(per_step_us, 90)), 2),
        "graph_only_ms_per_step": round(graph_ms, 5),
        "eager_only_ms_per_step": round(eager_ms, 5),
        "other_launch": {"launch": other, "ms_per_step": round(other_ms, 5), "step_us": round(other_ms * 1e3, 2),
                         "value": round(total / (other_ms * 1e-3) / 1e9, 2)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0, 1/fan_in) weights, N(0,1) target features, uniform token ids)",
        "config": {
            "workload": f"DFlash drafter block step + acceptance, real dims (5 layers, n_embd 6656, heads 32/8, "
                        f"head_dim 128, n_ff 19968, window 2048, block 16, vocab 8192), {wdt} weights, {rdt} ring, "
                        f"batch {B}, n_past {n_pasts}" + (f", block width {g}" if g != 16 else "")
                        + (f", drafts sampled at temperature {temp}" if temp > 0 else "")
                        + (", paged KV (128-slot pages, shuffled block tables)" if paged else ""),
            "batch": B,
            "block_width": g,
            "temperature": temp,
            "paged_kv": paged,
            "path": "persistent" if dr.step_path(B) == _lib.PATH_PERSISTENT else "kernels",
            "launch": args.launch,
            "algorithmic_bytes_per_step": total,
            "weight_bytes_per_step": nb["weights"],
            "ring_bytes_per_step": nb["ring"],
        },
        "roofline": {
            "kernel": "gate/up GEMV + SwiGLU (layer 0)",
            "bound": "hbm",
            "achieved": round(gu_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(gu_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": gu_bytes,
        },
        "accept": {"planted_mismatch_per_step": True, "last_step_n_ok_equals_planted": accept_ok},
        "context": PAGE_CONTEXT,
        "setup_s": round(setup_s, 1),
    }
    if T_inj:
        line["config"]["workload"] += f", {T_inj} positions injected before every step"
        line["config"]["inject_bytes_per_step"] = ib["total"]
        line["inject"] = {
            "positions": T_inj,
            "inject_us": round(inj["inject_us"], 2),
            "encode_us": round(inj["encode_us"], 2),
            "encode_tflops": round(ib["flops_encode"] / (inj["encode_us"] * 1e-6) / 1e12, 1),
            "inject_gbs": round(ib["total"] / (inj["inject_us"] * 1e-6) / 1e9, 1),
            "block_step_us_est": round(ms * 1e3 - inj["inject_us"], 2),
        }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(
            shape, raw, wdt, rdt, n_pasts[0], step_bytes(shape, wdt, rdt, n_vis[:1])["total"] + (ib["total"] if ib else 0),
            inject_feats=synth.features(shape, T_inj, fdt, seed=0, tag="bench.inject0") if T_inj else None,
            block_width=g)
    else:
        line["cpu_baseline"] = None
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dr.device).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = n
    graph.close()
    for sg in step_graphs:
        sg.close()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
