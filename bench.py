"""Throughput of the multi-LoRA metadata + shrink + expand step on one MI355X.

A step is one pass of the whole path (grouping metadata, shrink, expand) over
one synthetic batch, through lora_fused_step: one launch on small batches
(up to 512 token slots with few adapter outputs; the decode workload), else
lora_prepare_and_shrink and lora_expand.  The same step as three calls is
reported next to it.  Inputs are resident in HBM before timing starts.  To keep
the 256 MB Infinity Cache from serving repeats, R copies of every buffer (at
least 1 GiB in total) are rotated: one HIP graph holds consecutive steps, each
on the next copy in turn (at least 16 steps, so that a replay's fixed cost is
spread thin; a copy comes round again only after the others), and the timed
steps start on the copies the warm-up touched longest ago.  Per-kernel launch
durations for the roofline figure are measured the same way (a graph of at
least 32 launches of one kernel, over enough copies that the kernel's own
buffers span 1 GiB), with HIP events on the stream the graph is replayed on;
the roofline names the kernel of the step that takes the longest.  The CPU
oracle is timed on the host's cores on the same batch, as a reported baseline.

Prints exactly one JSON line on stdout (progress goes to stderr).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth
CPU_RUN_S = 3.0          # each CPU baseline run repeats full batches for about this long
CPU_MAX_THREADS = 16     # the host share of one GPU on the box
ROTATE_BYTES = 1 << 30
ROTATE_CAP = 48 << 30    # device memory the rotated copies may take in all
ROTATE_MAX_SETS = 512
# A graph cycles through its copies until it holds at least this many launch
# groups, so that the fixed cost of a replay is spread over many of them (a
# copy comes round again only after the others, which span ROTATE_BYTES).
MIN_GRAPH_STEPS = 16
MIN_GRAPH_LAUNCHES = 32
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "segmented_rank_gemm_amd", "csrc")
# sources a kernel's measured traffic depends on
KERNEL_SOURCES = {
    "lora_expand": ["expand.hip", "device_common.hpp"],
    "lora_shrink": ["shrink.hip", "device_common.hpp", "metadata_group.hpp"],
    "lora_prepare_metadata": ["metadata.hip", "device_common.hpp", "metadata_group.hpp"],
    "lora_fused_step": ["token_step.hip", "device_common.hpp", "metadata_group.hpp"],
}


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none for this kernel and workload or the kernel changed since."""
    path = os.path.join(PROFILES, f"{kernel}.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: 200 graph "
                    "replays' worth)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=1, help="workload index 0..4 (default 1: "
                    "Llama-2-7B qkv decode, rank 8)")
    ap.add_argument("--all", action="store_true", help="one line per workload 1..4")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rotate", type=int, default=None, help="buffer copies (default: >= 1 GiB)")
    ap.add_argument("--kernel-reps", type=int, default=50,
                    help="graph replays per single-kernel timing")
    ap.add_argument("--rules", action="store_true",
                    help="use the library's size rules for the part count and the expand's "
                    "launch choices instead of the measured table (segmented_rank_gemm_amd/"
                    "tuning_table.json)")
    ap.add_argument("--layers", type=int, default=32,
                    help="layers of the layer-stack timing (one metadata step, then shrink + "
                    "expand per layer on its own weights and activations; 0 skips it)")
    return ap.parse_args()


class Sets:
    """R device copies of one workload's buffers, plus the per-copy metadata;
    every expand call takes the given launch choices."""

    def __init__(self, w, R, num_splits, expand_cfg=None, start_delay_ns=None, part_sums=False,
                 batch_order_shrink=False, y_delay_ns=None):
        import torch

        import segmented_rank_gemm_amd as srg
        from workloads.device import to_dev_bf16

        self.w, self.R, self.num_splits = w, R, num_splits
        self.expand_cfg = expand_cfg
        self.start_delay_ns = start_delay_ns  # None: the library's default
        self.y_delay_ns = y_delay_ns
        self.part_sums = bool(part_sums)
        self.batch_order_shrink = bool(batch_order_shrink)
        T, maxT = w.num_tokens, w.max_tokens
        base = dict(
            mapping=torch.from_numpy(w.mapping.astype("int32")).cuda(),
            x=to_dev_bf16(w.x[:maxT]),
            y=to_dev_bf16(w.y0[:maxT]),
            a=[to_dev_bf16(a) for a in w.lora_a],
            b=[to_dev_bf16(b) for b in w.lora_b],
        )
        self.base = base
        self.sets = []
        self.T = T
        # one workspace serves every copy: the calls are ordered on one stream
        self.workspace = srg.fused_step_workspace(maxT, w.max_loras, w.num_slices, w.rank)
        self.one_launch = srg.lora_fused_step_launches(maxT, w.max_loras, w.num_slices,
                                                       w.rank) == 1
        self.grow(R)

    def grow(self, R):
        """Add copies up to R in total; the metadata of new copies is computed."""
        import torch

        import segmented_rank_gemm_amd as srg
        w, base, maxT = self.w, self.base, self.w.max_tokens
        while len(self.sets) < R:
            s = dict(
                mapping=base["mapping"].clone(), x=base["x"].clone(), y=base["y"].clone(),
                a=[t.clone() for t in base["a"]], b=[t.clone() for t in base["b"]],
                meta=srg.LoraMeta(maxT, w.max_loras),
                buf=torch.zeros((self.num_splits, w.num_slices, maxT, w.rank),
                                dtype=torch.float32, device="cuda"),
            )
            self.sets.append(s)
            self.metadata(len(self.sets) - 1)
        self.R = len(self.sets)
        torch.cuda.synchronize()

    def metadata(self, r, stream=None):
        import segmented_rank_gemm_amd as srg
        s = self.sets[r]
        srg.lora_prepare_metadata(s["mapping"], self.T, s["meta"], stream)

    def shrink(self, r, stream=None):
        import segmented_rank_gemm_amd as srg
        s = self.sets[r]
        srg.lora_shrink(s["x"], s["a"], float(self.w.scale), s["buf"], self.num_splits, s["meta"],
                        stream)

    def prep_shrink(self, r, stream=None):
        """Metadata and shrink of copy r in one call (lora_prepare_and_shrink)."""
        import segmented_rank_gemm_amd as srg
        s = self.sets[r]
        srg.lora_prepare_and_shrink(s["mapping"], self.T, s["x"], s["a"], float(self.w.scale),
                                    s["buf"], self.num_splits, s["meta"], stream)

    def expand(self, r, stream=None):
        import segmented_rank_gemm_amd as srg
        s = self.sets[r]
        srg.lora_expand(s["buf"], self.num_splits, s["b"], s["y"], s["meta"], stream,
                        config=self.expand_cfg)

    def layer(self, r, meta_r, stream=None):
        """Shrink + expand on copy r (one layer's weights and activations) with the
        metadata computed on copy meta_r."""
        import segmented_rank_gemm_amd as srg
        s, m = self.sets[r], self.sets[meta_r]["meta"]
        srg.lora_shrink(s["x"], s["a"], float(self.w.scale), s["buf"], self.num_splits, m, stream)
        srg.lora_expand(s["buf"], self.num_splits, s["b"], s["y"], m, stream,
                        config=self.expand_cfg)

    def fused(self, r, stream=None, meta_r=None):
        """The whole path in one call (lora_fused_step), writing copy meta_r's
        metadata (default: copy r's)."""
        import segmented_rank_gemm_amd as srg
        s = self.sets[r]
        m = s["meta"] if meta_r is None else self.sets[meta_r]["meta"]
        srg.lora_fused_step(s["mapping"], self.T, s["x"], s["a"], s["b"], float(self.w.scale),
                            s["buf"], self.num_splits, s["y"], m, self.workspace, stream=stream,
                            expand_config=self.expand_cfg, start_delay_ns=self.start_delay_ns,
                            part_sums=self.part_sums,
                            batch_order_shrink=self.batch_order_shrink,
                            y_delay_ns=self.y_delay_ns)

    def step(self, r, stream=None):
        """The whole path: lora_fused_step."""
        self.fused(r, stream)

    def step2(self, r, stream=None):
        """The whole path as lora_prepare_and_shrink + lora_expand."""
        self.prep_shrink(r, stream)
        self.expand(r, stream)

    def step3(self, r, stream=None):
        """The whole path as three calls: metadata, shrink, expand."""
        self.metadata(r, stream)
        self.shrink(r, stream)
        self.expand(r, stream)


def set_bytes(w, num_splits):
    maxT = w.max_tokens
    return (maxT * w.hidden * 2 + maxT * w.n_total * 2 + w.num_tokens * 4 + maxT * 4
            + sum(a.nbytes for a in w.lora_a) + sum(b.nbytes for b in w.lora_b)
            + num_splits * w.num_slices * maxT * w.rank * 4)


def kernel_set_bytes(w, num_splits):
    """Bytes of one buffer copy that each kernel touches (its share of set_bytes)."""
    maxT = w.max_tokens
    buf = num_splits * w.num_slices * maxT * w.rank * 4
    shrink = maxT * w.hidden * 2 + sum(a.nbytes for a in w.lora_a) + buf
    expand = maxT * w.n_total * 2 + sum(b.nbytes for b in w.lora_b) + buf
    return {"metadata": w.num_tokens * 4 + maxT * 4, "shrink": shrink, "expand": expand,
            "pair": shrink + expand - buf}


def rotation(nbytes, set_total, floor):
    """Copies needed for nbytes per copy to span ROTATE_BYTES, within ROTATE_CAP of
    memory and ROTATE_MAX_SETS launches per graph."""
    want = max(floor, math.ceil(ROTATE_BYTES / max(nbytes, 1)))
    return max(floor, min(want, ROTATE_CAP // max(set_total, 1), ROTATE_MAX_SETS))


def capture(fn_list):
    """One HIP graph running the given launches in order on a side stream."""
    import torch
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        cur = torch.cuda.current_stream()
        for f in fn_list:
            f(cur)
    torch.cuda.synchronize()
    return g


def time_graph(g, reps):
    """Average seconds per replay, HIP events on the replay stream."""
    import torch
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        g.replay()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / reps


def _cpu_run(w, threads, min_s):
    """Full oracle batches (metadata + shrink + expand, fp64) repeated for at
    least min_s seconds (and at least one batch): tokens per second."""
    import oracle
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.run_step(w, num_threads=threads)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return w.num_tokens * n / el, n, el


def cpu_baseline(w):
    """The oracle on the host: median of 3 runs on the threads the box gives one
    GPU (at most 16, fewer if the process may use fewer cores), after a warm-up,
    and one single-thread run."""
    import oracle
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(CPU_MAX_THREADS, avail))
    oracle.run_step(w, num_threads=threads)  # warm-up
    runs = [_cpu_run(w, threads, CPU_RUN_S) for _ in range(3)]
    rates = sorted(r[0] for r in runs)
    single = _cpu_run(w, 1, CPU_RUN_S)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    batches = sum(r[1] for r in runs)
    secs = sum(r[2] for r in runs)
    return dict(value=rates[1], unit="tokens/s", cores=threads, kind="oracle",
                sample=f"3 runs of full batches of {w.num_tokens} tokens (metadata+shrink+expand, "
                       f"fp64), {batches} batches in {secs:.1f} s, median of the three; "
                       f"{model}".strip(),
                runs_tokens_per_s=rates, single_thread_tokens_per_s=single[0],
                host_cores_visible=os.cpu_count(), cores_usable=avail)


def run_config(idx, args):
    import torch

    import segmented_rank_gemm_amd as srg
    from segmented_rank_gemm_amd import measure
    from workloads import WORKLOADS, make_workload, workload_stats

    log(f"[bench] workload {idx} ({WORKLOADS[idx]['name']}): generating inputs")
    w = make_workload(idx)
    st = workload_stats(w)
    from segmented_rank_gemm_amd.tuning import plan
    rule_splits = srg.lora_shrink_default_splits(w.hidden, w.max_tokens, w.max_loras,
                                                 w.num_slices, w.rank)
    pl = plan(w.hidden, w.max_tokens, w.max_loras, w.slices, w.rank)
    if args.rules:
        pl = {"num_splits": rule_splits, "expand": srg.ExpandConfig(), "start_delay_ns": None,
              "y_delay_ns": None, "part_sums": False, "batch_order_shrink": False,
              "source": "size rule"}
    splits = pl["num_splits"]
    expand_cfg = pl["expand"] or srg.ExpandConfig()
    sb = set_bytes(w, splits)
    R = args.rotate or max(2, math.ceil(ROTATE_BYTES / sb))
    log(f"[bench] {R} rotated buffer sets of {sb / 1e6:.1f} MB, {splits} shrink parts")
    sets = Sets(w, R, splits, expand_cfg, pl["start_delay_ns"], pl["part_sums"],
                pl["batch_order_shrink"], pl["y_delay_ns"])

    # eager pass on every set so the metadata exists before single-kernel graphs replay
    for r in range(R):
        sets.step(r)
    torch.cuda.synchronize()

    G = R * max(1, math.ceil(MIN_GRAPH_STEPS / R))  # steps per graph, copies in turn
    steps = args.steps if args.steps is not None else R * 200
    warm = args.warmup if args.warmup is not None else R * 20
    # warm-up on copies 0, 1, ...; the timed steps start where the warm-up
    # stopped, so with fewer steps than copies none of them reuses a copy the
    # warm-up has just brought into the caches
    off = warm % R
    g_warm = capture([lambda s, r=r: sets.step(r % R, s) for r in range(G)])
    g_step = capture([lambda s, r=r: sets.step((off + r) % R, s) for r in range(G)])
    full, rem = divmod(steps, G)
    g_rem = (capture([lambda s, r=r: sets.step((off + full * G + r) % R, s) for r in range(rem)])
             if rem else None)
    wfull, wrem = divmod(warm, G)
    log(f"[bench] warmup {warm} steps")
    for _ in range(wfull):
        g_warm.replay()
    if wrem:
        capture([lambda s, r=r: sets.step(r % R, s) for r in range(wrem)]).replay()
    torch.cuda.synchronize()
    del g_warm

    log(f"[bench] timing {steps} steps from copy {off}")
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(full):
        g_step.replay()
    if g_rem is not None:
        g_rem.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = start.elapsed_time(end) / 1e3
    step_s = wall / steps
    del g_step, g_rem

    # single-kernel graphs: average launch duration of each kernel over enough
    # copies that the kernel's own buffers span ROTATE_BYTES (so the Infinity
    # Cache cannot serve a repeat), more copies than the step needs when the
    # kernel touches only part of a set
    reps = args.kernel_reps
    log("[bench] per-kernel timing")
    kb = kernel_set_bytes(w, splits)
    # (the metadata kernel reads a few KB per copy: it is timed over the step's copies)
    # (--rotate fixes the copies for every kernel, e.g. for short counter runs)
    kb["prepare_and_shrink"] = kb["shrink"] + kb["metadata"]
    kb["step3"] = sb
    kb["step2"] = sb
    kb["fused_step"] = sb
    rot = {k: (R if k in ("metadata", "step3", "step2", "fused_step") or args.rotate
               else rotation(kb[k], sb, R)) for k in kb}
    sets.grow(max(rot.values()))
    per = {}
    fns = {"metadata": sets.metadata, "shrink": sets.shrink, "expand": sets.expand,
           "prepare_and_shrink": sets.prep_shrink, "fused_step": sets.fused,
           "pair": lambda r, s: (sets.shrink(r, s), sets.expand(r, s)), "step3": sets.step3,
           "step2": sets.step2}
    for name in ("metadata", "shrink", "prepare_and_shrink", "expand", "fused_step", "pair",
                 "step2", "step3"):
        n = rot[name]
        m = n * max(1, math.ceil(MIN_GRAPH_LAUNCHES / n))  # launch groups per graph
        g = capture([lambda s, r=r, f=fns[name]: f(r % n, s) for r in range(m)])
        per[name] = time_graph(g, reps) / m
        del g
    pair_s = per.pop("pair")
    step3_s = per.pop("step3")
    step2_s = per.pop("step2")

    # large batches: the same step with the large-batch options the table did
    # not choose, where they apply (measured beside the chosen one; same bits)
    options = {}
    if not sets.one_launch and w.max_tokens > 512:
        variants = [("batch_order_shrink", dict(batch_order_shrink=not sets.batch_order_shrink,
                                                part_sums=False))]
        if w.rank >= 32 and splits >= 2:
            variants.append(("part_sums", dict(batch_order_shrink=False,
                                               part_sums=not sets.part_sums)))
        chosen = (sets.batch_order_shrink, sets.part_sums)
        n = rot["fused_step"]
        m = n * max(1, math.ceil(MIN_GRAPH_LAUNCHES / n))
        for name, flags in variants:
            sets.batch_order_shrink, sets.part_sums = flags["batch_order_shrink"], flags["part_sums"]
            g = capture([lambda s, r=r: sets.fused(r % n, s) for r in range(m)])
            options[f"{name}={'on' if flags[name] else 'off'}"] = time_graph(g, reps) / m * 1e6
            del g
        sets.batch_order_shrink, sets.part_sums = chosen
        options["as_chosen"] = per["fused_step"] * 1e6

    # V0-style input: the same batch regrouped by adapter (each group one
    # contiguous run), through the general metadata kernel and the one-pass
    # grouped one (same outputs)
    import numpy as np
    ids = np.where((w.mapping >= -1) & (w.mapping < w.max_loras), w.mapping, -1)
    gmap = torch.from_numpy(w.mapping[np.argsort(ids, kind="stable")].astype("int32")).cuda()
    gmaps = [gmap.clone() for _ in range(R)]
    grouped = {}
    for name, f in (("lora_prepare_metadata", srg.lora_prepare_metadata),
                    ("lora_prepare_metadata_grouped", srg.lora_prepare_metadata_grouped)):
        m = R * max(1, math.ceil(MIN_GRAPH_LAUNCHES / R))
        g = capture([lambda s, r=r, f=f: f(gmaps[r % R], sets.T, sets.sets[r % R]["meta"], s)
                     for r in range(m)])
        grouped[name + "_us"] = time_graph(g, reps) / m * 1e6
        del g
    del gmaps
    # (the copies' metadata is the regrouped batch's now: recompute it)
    for r in range(sets.R):
        sets.metadata(r)
    torch.cuda.synchronize()

    # layer stack: one metadata step serves a model's L LoRA layers of this
    # shape, each with its own weights, activations and outputs.  Stacks are
    # rotated like the steps (each stack takes L copies and computes its
    # metadata on its first).  One-launch sizes: every layer is a
    # lora_fused_step; otherwise the first layer groups the batch in its
    # lora_prepare_and_shrink and the others run lora_shrink + lora_expand on it.
    stack = None
    L = args.layers
    if L > 0:
        K = max(1, math.ceil(max(R, rot["expand"]) / L))
        log(f"[bench] layer stack: {K} stacks of {L} layers")
        sets.grow(K * L)
        calls = []
        for k in range(K):
            m = k * L
            if sets.one_launch:
                calls += [lambda s, r=m + l, m=m: sets.fused(r, s, meta_r=m) for l in range(L)]
            else:
                calls.append(lambda s, m=m: (sets.prep_shrink(m, s), sets.expand(m, s)))
                calls += [lambda s, r=m + l, m=m: sets.layer(r, m, s) for l in range(1, L)]
        g = capture(calls)
        t_stack = time_graph(g, max(2, reps // 10)) / K
        del g
        stack = {
            "layers": L, "rotated_stacks": K, "us": t_stack * 1e6, "us_per_layer": t_stack / L * 1e6,
            "calls": ("lora_fused_step per layer" if sets.one_launch else
                      "lora_prepare_and_shrink + lora_expand, then lora_shrink + lora_expand"),
            "layer_tokens_per_s": w.num_tokens * L / t_stack,
        }

    # practical ceilings for the expand's bytes, same rotation: a copy between
    # two buffers, and an in-place update of one (the expand's access pattern)
    cb = (st["expand_bytes"] // 2) // 16 * 16
    Rc = rot["expand"]
    srcs = [torch.empty(cb, dtype=torch.uint8, device="cuda") for _ in range(Rc)]
    dsts = [torch.empty(cb, dtype=torch.uint8, device="cuda") for _ in range(Rc)]
    g_copy = capture([lambda s, r=r: measure.lora_stream_copy(srcs[r], dsts[r], s) for r in range(Rc)])
    copy_s = time_graph(g_copy, reps) / Rc
    g_upd = capture([lambda s, r=r: measure.lora_stream_update(srcs[r], s) for r in range(Rc)])
    upd_s = time_graph(g_upd, reps) / Rc
    del g_copy, g_upd, srcs, dsts

    # the kernels of the step with their algorithmic bytes per launch; the
    # roofline is that of the one that takes the longest
    if sets.one_launch:
        step_kernels = {"lora_fused_step": (per["fused_step"], st["total_bytes"])}
    else:
        step_kernels = {
            "lora_prepare_metadata": (per["metadata"], st["index_bytes"]),
            "lora_shrink": (per["shrink"], st["shrink_bytes"]),
            "lora_expand": (per["expand"], st["expand_bytes"]),
        }
    dom = max(step_kernels, key=lambda k: step_kernels[k][0])
    dom_s, dom_bytes = step_kernels[dom]
    achieved = dom_bytes / dom_s / 1e9
    out = {
        "metric": "fused shrink+expand tokens/s and achieved HBM GB/s (% of peak), "
                  "Llama-2-7B qkv r=8",
        "value": w.num_tokens / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[idx]["name"], "num_tokens": w.num_tokens,
            "active_tokens": st["active_tokens"], "hidden": w.hidden, "slices": w.slices,
            "rank": w.rank, "max_loras": w.max_loras, "active_adapters": st["active_adapters"],
            "scale": w.scale, "accumulate": "fp32", "shrink_parts": splits,
            "shrink_parts_from": pl["source"], "shrink_parts_rule": rule_splits,
            "expand_config": expand_cfg.as_dict(), "expand_config_from": pl["source"],
            "start_delay_ns": pl["start_delay_ns"] if pl["start_delay_ns"] is not None else "default",
            "y_delay_ns": pl["y_delay_ns"] if pl["y_delay_ns"] is not None else "default",
            "part_sums": pl["part_sums"], "batch_order_shrink": pl["batch_order_shrink"],
            "rotated_sets": R, "rotated_sets_per_kernel": rot, "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "kernel": dom, "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(dom, WORKLOADS[idx]["name"]),
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_us": dom_s * 1e6,
            "step_kernels_us": {k: v[0] * 1e6 for k, v in step_kernels.items()},
        },
        "step": {
            "calls": "lora_fused_step",
            "launches": ("one" if sets.one_launch else
                         "lora_prepare_and_shrink (one or two kernels) + lora_expand"),
            "gpu_event_ms_per_step": gpu_s / steps * 1e3,
            "algorithmic_bytes": st["total_bytes"],
            "achieved_GBs": st["total_bytes"] / step_s / 1e9,
            "frac_of_peak": st["total_bytes"] / step_s / 1e9 / HBM_PEAK_GBS,
        },
        "kernels_us": {k: v * 1e6 for k, v in per.items()},
        "step_two_calls": {
            "calls": "lora_prepare_and_shrink + lora_expand",
            "us": step2_s * 1e6, "tokens_per_s": w.num_tokens / step2_s,
        },
        "step_three_calls": {
            "calls": "lora_prepare_metadata + lora_shrink + lora_expand",
            "us": step3_s * 1e6, "tokens_per_s": w.num_tokens / step3_s,
        },
        "shrink_expand_pair": {
            "us": pair_s * 1e6,
            "tokens_per_s": w.num_tokens / pair_s,
            "achieved_GBs": (st["shrink_bytes"] + st["expand_bytes"]) / pair_s / 1e9,
            "frac_of_peak": (st["shrink_bytes"] + st["expand_bytes"]) / pair_s / 1e9 / HBM_PEAK_GBS,
        },
        "layer_stack": stack,
        "step_us_by_large_batch_option": options or None,
        "grouped_input": dict(grouped, batch="the same batch regrouped by adapter (V0-style)"),
        "copy_ceiling": {"bytes_read_plus_written": 2 * cb, "us": copy_s * 1e6,
                         "GBs": 2 * cb / copy_s / 1e9},
        "update_ceiling": {"bytes_read_plus_written": 2 * cb, "us": upd_s * 1e6,
                           "GBs": 2 * cb / upd_s / 1e9},
    }
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(w)
    else:
        out["cpu_baseline"] = None
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the op shards "
              "per token or per output column without any exchange, and no multi-GPU path is "
              "built here", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    configs = [1, 2, 3, 4] if args.all else [args.config]
    for i in configs:
        print(json.dumps(run_config(i, args)), flush=True)


if __name__ == "__main__":
    main()
