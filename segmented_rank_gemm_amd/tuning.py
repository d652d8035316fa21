"""Per-shape launch choices of the multi-LoRA path: a measured table.

vLLM PR #11613 "[Do Not Merge] - LoRA V1 Reference PR" lists autotuning the V1
LoRA kernels among the follow-up items of its split plan.  The choices that
change how the work is cut but never the result are:

* ``num_splits``: the number of contiguous hidden-dimension parts the shrink
  computes separately and the expand sums.  More parts spread a batch over more
  workgroups; fewer mean fewer partial rows to read and less start-up per
  unit.  It fixes the ``buf`` shape, so a captured graph keeps the value it
  was captured with.
* the expand's launch choices (``lora_expand_config_t``): the column-range
  length, the unit order and the workgroups per CU its grid is sized for.
* on the one-launch path, how long the expand workgroups hold their own B and
  y loads back so that the shrink workgroups' loads are served first
  (``lora_step_options_t.start_delay_ns``, ``y_delay_ns``); on the
  multi-launch path for large
  rank-32/64 batches, whether the shrink sums the parts for the expand
  (``part_sums``); for large batches, whether the shrink runs in batch order
  beside the metadata (``batch_order_shrink``: faster on batches of request
  runs, so it is measured on the workload's own batch).

Where the optimum lies depends on how the batch's tiles round against the
compute units, and the tile count is a property of the batch's adapter mix,
known only once the batch is grouped, so the library's built-in rules are a
function of the sizes alone and this module settles each shape by timing the
candidates on a representative batch.  ``tuning_table.json`` (next to this
file) holds the result per shape, written by ``python -m
segmented_rank_gemm_amd.tuning --generate`` on the GPU; ``plan`` returns a
shape's entry (or the rules), and the binding's ``lora_expand`` /
``lora_fused_step`` use a shape's expand choices and hold-off by default.

The timing helpers are host-side utilities for an offline step, not part of
the path: they only call the library's entry points, allocate their own copies
of the operands with torch, synchronise, and never write the caller's tensors.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from typing import Dict, Iterable, List, Optional, Sequence

import torch

from . import (LORA_MAX_SPLITS, ExpandConfig, LoraMeta, lora_expand, lora_shrink,
               lora_shrink_default_splits)

CHUNK = 64  # hidden elements per step of the shrink kernels; a part is a multiple of it
_GRID = (1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16)


def candidate_splits(hidden: int, max_tokens: int, max_loras: int, num_slices: int,
                     rank: int) -> List[int]:
    """The part counts worth timing for a shape: 1-8, 10, 12, 16 and the size
    rule's own value, none larger than the number of 64-element chunks of the
    hidden dimension (a further part would be empty) or LORA_MAX_SPLITS."""
    chunks = max(1, math.ceil(hidden / CHUNK))
    limit = min(chunks, LORA_MAX_SPLITS)
    out = {v for v in _GRID if v <= limit}
    d = lora_shrink_default_splits(hidden, max_tokens, max_loras, num_slices, rank)
    if 1 <= d <= LORA_MAX_SPLITS:
        out.add(d)
    return sorted(out)


def _graph_seconds(launch, copies: int, reps: int) -> float:
    """Average seconds of one launch group, from a HIP graph of `copies` groups
    (one per operand copy) replayed `reps` times, timed with events on the
    replay stream."""
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        cur = torch.cuda.current_stream()
        for i in range(copies):
            launch(i, cur)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(s)
    for _ in range(reps):
        g.replay()
    t1.record(s)
    t1.synchronize()
    del g
    return t0.elapsed_time(t1) / 1e3 / (reps * copies)


def tune_shrink_splits(x: torch.Tensor, lora_a: Sequence[torch.Tensor],
                       lora_b: Sequence[torch.Tensor], y: torch.Tensor, scale: float,
                       meta: LoraMeta, candidates: Optional[Iterable[int]] = None,
                       rotate_bytes: int = 1 << 30, reps: int = 20) -> Dict[str, object]:
    """Time lora_shrink + lora_expand for each candidate ``num_splits`` on one batch.

    x, lora_a, lora_b, y as for ``lora_shrink`` / ``lora_expand``; ``meta`` must
    already hold the batch's grouping (``lora_prepare_metadata``).  The operands
    are copied as many times as it takes for the copies to span
    ``rotate_bytes`` (so that the Infinity Cache cannot serve repeats), and each
    candidate is timed as a graph of one pair per copy.  Returns
    ``{"best": n, "default": d, "us": {n: microseconds per pair}}``.
    """
    S = len(lora_a)
    _, rank, hidden = (int(v) for v in lora_a[0].shape)
    maxT, L = meta.max_tokens, meta.max_loras
    default = lora_shrink_default_splits(hidden, maxT, L, S, rank)
    cands = sorted(set(candidates)) if candidates is not None else candidate_splits(
        hidden, maxT, L, S, rank)
    if not cands or any(c < 1 or c > LORA_MAX_SPLITS for c in cands):
        raise ValueError(f"candidates must lie in [1, {LORA_MAX_SPLITS}]: {cands}")
    if reps < 1:
        raise ValueError("reps must be at least 1")

    nbytes = (x.numel() * x.element_size() + y.numel() * y.element_size()
              + sum(t.numel() * t.element_size() for t in lora_a)
              + sum(t.numel() * t.element_size() for t in lora_b)
              + max(cands) * S * maxT * rank * 4)
    copies = max(2, math.ceil(rotate_bytes / max(nbytes, 1)))
    ops = [dict(x=x.clone(), a=[t.clone() for t in lora_a], b=[t.clone() for t in lora_b],
                y=y.clone()) for _ in range(copies)]
    us: Dict[int, float] = {}
    for n in cands:
        bufs = [torch.empty((n, S, maxT, rank), dtype=torch.float32, device=x.device)
                for _ in range(copies)]

        def pair(i, stream, n=n, bufs=bufs):
            o = ops[i]
            lora_shrink(o["x"], o["a"], scale, bufs[i], n, meta, stream)
            lora_expand(bufs[i], n, o["b"], o["y"], meta, stream, config=None)

        for i in range(copies):  # eager pass first (and a check that the launch is accepted)
            pair(i, None)
        torch.cuda.synchronize()
        us[n] = _graph_seconds(pair, copies, reps) * 1e6
        del bufs
    del ops
    torch.cuda.synchronize()
    best = min(us, key=us.get)
    return {"best": best, "default": default, "us": us}


# ------------------------------------------------------------------ table

TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuning_table.json")
_table_cache: Optional[Dict[str, dict]] = None


def shape_key(hidden: int, max_tokens: int, max_loras: int, slices: Sequence[int],
              rank: int) -> str:
    """The table key of a shape: the sizes that fix the grids."""
    return (f"hidden={int(hidden)},max_tokens={int(max_tokens)},max_loras={int(max_loras)},"
            f"slices={'x'.join(str(int(n)) for n in slices)},rank={int(rank)}")


def load_table(path: str = TABLE_PATH) -> Dict[str, dict]:
    """The committed table ({} if there is none)."""
    global _table_cache
    if path == TABLE_PATH and _table_cache is not None:
        return _table_cache
    table = {}
    if os.path.exists(path):
        with open(path) as f:
            table = {e["key"]: e for e in json.load(f)["entries"]}
    if path == TABLE_PATH:
        _table_cache = table
    return table


def lookup(hidden: int, max_tokens: int, max_loras: int, slices: Sequence[int],
           rank: int) -> Optional[dict]:
    """The table's entry for a shape, or None."""
    return load_table().get(shape_key(hidden, max_tokens, max_loras, slices, rank))


def plan(hidden: int, max_tokens: int, max_loras: int, slices: Sequence[int],
         rank: int) -> dict:
    """Launch choices for a shape: the table's measured ones where the table
    has the shape, else the library's size rules.  Returns
    {"num_splits": n, "expand": ExpandConfig or None, "start_delay_ns": ns or None,
     "y_delay_ns": ns or None, "part_sums": bool, "batch_order_shrink": bool,
     "source": "table" | "size rule"}."""
    e = lookup(hidden, max_tokens, max_loras, slices, rank)
    if e is not None:
        delay, y_delay = e.get("start_delay_ns"), e.get("y_delay_ns")
        return {"num_splits": int(e["num_splits"]), "expand": ExpandConfig(**e["expand"]),
                "start_delay_ns": None if delay is None else int(delay),
                "y_delay_ns": None if y_delay is None else int(y_delay),
                "part_sums": bool(e.get("part_sums", False)),
                "batch_order_shrink": bool(e.get("batch_order_shrink", False)), "source": "table"}
    return {"num_splits": lora_shrink_default_splits(hidden, max_tokens, max_loras, len(slices),
                                                     rank),
            "expand": None, "start_delay_ns": None, "y_delay_ns": None, "part_sums": False,
            "batch_order_shrink": False, "source": "size rule"}


def _entry_for(lora_b: Sequence[torch.Tensor], num_splits: int, meta: LoraMeta) -> Optional[dict]:
    """The table entry with the call's max_tokens, max_loras, slices and rank
    whose part count is the call's (the expand reads that many parts; the
    hidden size does not reach it), or None."""
    slices = [int(b.shape[1]) for b in lora_b]
    rank = int(lora_b[0].shape[2])
    for e in load_table().values():
        sh = e.get("shape", {})
        if (sh.get("max_tokens") == meta.max_tokens and sh.get("max_loras") == meta.max_loras
                and sh.get("slices") == slices and sh.get("rank") == rank
                and e.get("num_splits") == int(num_splits)):
            return e
    return None


def expand_config_for(lora_b: Sequence[torch.Tensor], num_splits: int,
                      meta: LoraMeta) -> Optional[ExpandConfig]:
    """The table's expand choices for the call at hand, or None (the
    library's rules)."""
    e = _entry_for(lora_b, num_splits, meta)
    return None if e is None else ExpandConfig(**e["expand"])


def flag_for(name: str, lora_b: Sequence[torch.Tensor], num_splits: int, meta: LoraMeta) -> bool:
    """The table's yes/no choice `name` ("part_sums", "batch_order_shrink") for
    the call at hand (no when the table has none)."""
    e = _entry_for(lora_b, num_splits, meta)
    return bool(e is not None and e.get(name, False))


def start_delay_for(lora_b: Sequence[torch.Tensor], num_splits: int, meta: LoraMeta,
                    name: str = "start_delay_ns") -> Optional[int]:
    """The table's one-launch expand hold-off `name` ("start_delay_ns" before
    the B loads, "y_delay_ns" before the y loads) for the call at hand, in ns,
    or None (the library's default)."""
    e = _entry_for(lora_b, num_splits, meta)
    if e is None or e.get(name) is None:
        return None
    return int(e[name])


# (y hold-off, B hold-off) pairs timed for one-launch shapes, ns
_HOLD_CANDIDATES_NS = tuple((yd, bd) for yd in (0, 400, 600, 800, 1000, 1200)
                            for bd in (1600, 2000, 2200, 2400, 2600, 2800, 3200))


def _expand_candidates(rank: int) -> List[ExpandConfig]:
    out = [ExpandConfig()]  # the rules
    if rank <= 16:
        for cpr in (1, 2, 3, 4, 8):
            for order in (0, 1):
                out.append(ExpandConfig(cpr, order, 0))
    else:
        for cpr in (0, 4, 6, 8, 12, 16):
            for wpc in (1, 2, 3):
                for order in (0, 1):
                    out.append(ExpandConfig(cpr, order, wpc))
    return out


def tune_workload(w, reps: int = 20, log=print) -> dict:
    """Measure the launch choices for one workload's shape on its batch: the
    whole step (lora_fused_step: one launch where it applies, else
    lora_prepare_and_shrink + lora_expand), first over the part counts with
    the expand's rules, then over the expand's choices at the best part count.
    Graphs over copies of the operands spanning 1 GiB, events on the replay
    stream.  Returns the table entry."""
    from workloads.device import to_dev_bf16

    from . import fused_step_workspace, lora_fused_step, lora_fused_step_launches

    maxT, S, r = w.max_tokens, w.num_slices, w.rank
    rule = lora_shrink_default_splits(w.hidden, maxT, w.max_loras, S, r)
    ws = fused_step_workspace(maxT, w.max_loras, S, r)
    one_launch = lora_fused_step_launches(maxT, w.max_loras, S, r) == 1
    sums_possible = not one_launch and ws is not None  # the part sums' workspace
    base = dict(mapping=torch.from_numpy(w.mapping.astype("int32")).cuda(),
                x=to_dev_bf16(w.x[:maxT]), y=to_dev_bf16(w.y0[:maxT]),
                a=[to_dev_bf16(a) for a in w.lora_a], b=[to_dev_bf16(b) for b in w.lora_b])
    per_copy = (base["x"].numel() + base["y"].numel()) * 2 + sum(
        t.numel() * 2 for t in base["a"] + base["b"])
    copies = max(2, math.ceil((1 << 30) / per_copy))
    ops = [dict(mapping=base["mapping"].clone(), x=base["x"].clone(), y=base["y"].clone(),
                a=[t.clone() for t in base["a"]], b=[t.clone() for t in base["b"]],
                meta=LoraMeta(maxT, w.max_loras)) for _ in range(copies)]

    def time_step(n, cfg, delay=None, sums=False, batch=False, y_delay=None):
        bufs = [torch.empty((n, S, maxT, r), dtype=torch.float32, device="cuda")
                for _ in range(copies)]

        def step(i, stream):
            o = ops[i]
            lora_fused_step(o["mapping"], w.num_tokens, o["x"], o["a"], o["b"], float(w.scale),
                            bufs[i], n, o["y"], o["meta"], ws, stream=stream,
                            expand_config=cfg if cfg is not None else ExpandConfig(),
                            start_delay_ns=delay, part_sums=sums, batch_order_shrink=batch,
                            y_delay_ns=y_delay)

        for i in range(copies):
            step(i, None)
        torch.cuda.synchronize()
        t = _graph_seconds(step, copies, reps) * 1e6
        del bufs
        return t

    cands = candidate_splits(w.hidden, maxT, w.max_loras, S, r)
    if one_launch:
        cands = sorted({c for c in cands if c >= 4} | ({rule, 20, 24, 32} & set(range(1, 65))))
    # large batches: the grouped shrink after the metadata kernel, or the
    # batch-order shrink beside it (decided on this batch, then kept)
    batch_possible = not one_launch and maxT > 512
    batch = False
    us_splits = {}
    for n in cands:
        us_splits[n] = time_step(n, None)
        log(f"[tune] {w.name} splits={n}: {us_splits[n]:.2f} us")
    us_batch = {}
    if batch_possible:
        for n in cands:
            us_batch[n] = time_step(n, None, batch=True)
            log(f"[tune] {w.name} batch-order shrink, splits={n}: {us_batch[n]:.2f} us")
        if min(us_batch.values()) < min(us_splits.values()):
            batch = True
    best_n = min(us_batch, key=us_batch.get) if batch else min(us_splits, key=us_splits.get)
    us_expand = {}
    best_cfg = ExpandConfig()
    if not one_launch:
        for cfg in _expand_candidates(r):
            key = json.dumps(cfg.as_dict(), sort_keys=True)
            us_expand[key] = time_step(best_n, cfg, batch=batch)
            log(f"[tune] {w.name} splits={best_n} expand={key}: {us_expand[key]:.2f} us")
        best_key = min(us_expand, key=us_expand.get)
        best_cfg = ExpandConfig(**json.loads(best_key))
    # the same two sweeps with the shrink summing the parts for the expand
    us_sums = {}
    best_sums = False
    if sums_possible:
        us_sums_splits = {}
        for n in cands:
            if n >= 2:
                us_sums_splits[n] = time_step(n, None, sums=True)
                log(f"[tune] {w.name} part sums, splits={n}: {us_sums_splits[n]:.2f} us")
        sn = min(us_sums_splits, key=us_sums_splits.get)
        for cfg in _expand_candidates(r):
            key = json.dumps(cfg.as_dict(), sort_keys=True)
            us_sums[key] = time_step(sn, cfg, sums=True)
            log(f"[tune] {w.name} part sums, splits={sn} expand={key}: {us_sums[key]:.2f} us")
        skey = min(us_sums, key=us_sums.get)
        if us_sums[skey] < min(us_expand.values()):
            best_sums, best_n, best_cfg = True, sn, ExpandConfig(**json.loads(skey))
            us_expand = dict(us_expand, **{"part sums " + k: v for k, v in us_sums.items()})
    # the one-launch path's expand hold-offs (y, then B), at the best part
    # count (None: the library's defaults from the shrink's per-workgroup bytes)
    us_delay = {}
    best_delay = best_y_delay = None
    if one_launch:
        us_delay["default"] = us_splits[best_n]
        for yd, bd in _HOLD_CANDIDATES_NS:
            key = f"{yd},{bd}"
            us_delay[key] = time_step(best_n, None, bd, y_delay=yd)
            log(f"[tune] {w.name} splits={best_n} y_delay_ns={yd} start_delay_ns={bd}: "
                f"{us_delay[key]:.2f} us")
        best_key = min(us_delay, key=us_delay.get)
        if best_key != "default":
            best_y_delay, best_delay = (int(v) for v in best_key.split(","))
    best_us = min(us_expand.values()) if us_expand else (
        min(us_delay.values()) if us_delay else us_splits[best_n])
    del ops
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {
        "key": shape_key(w.hidden, maxT, w.max_loras, w.slices, r),
        "shape": {"hidden": int(w.hidden), "max_tokens": int(maxT), "max_loras": int(w.max_loras),
                  "slices": [int(n) for n in w.slices], "rank": int(r)},
        "workload": w.name,
        "num_splits": int(best_n),
        "expand": best_cfg.as_dict(),
        "start_delay_ns": best_delay,
        "y_delay_ns": best_y_delay,
        "part_sums": best_sums,
        "batch_order_shrink": batch and not best_sums,
        "step_us": round(best_us, 3),
        "rule": {"num_splits": int(rule), "step_us": round(us_splits.get(rule, float("nan")), 3)},
        "step_us_by_splits": {str(k): round(v, 3) for k, v in us_splits.items()},
        "step_us_by_splits_batch_order": {str(k): round(v, 3) for k, v in us_batch.items()},
        "step_us_by_expand": {k: round(v, 3) for k, v in us_expand.items()},
        "step_us_by_hold_offs_ns": {k: round(v, 3) for k, v in us_delay.items()},
        "step_us_with_part_sums": {k: round(v, 3) for k, v in us_sums.items()},
    }


def generate(configs: Sequence[int], path: str = TABLE_PATH, reps: int = 20) -> None:
    """Tune the given benchmark workloads and write the table (entries for
    other shapes already in the file are kept)."""
    from workloads import make_workload

    table = dict(load_table(path)) if os.path.exists(path) else {}
    for c in configs:
        w = make_workload(c)
        e = tune_workload(w, reps=reps, log=lambda *a: print(*a, file=sys.stderr, flush=True))
        table[e["key"]] = e
    out = {"device": torch.cuda.get_device_properties(0).gcnArchName,
           "generated_by": "python -m segmented_rank_gemm_amd.tuning --generate",
           "date": time.strftime("%Y-%m-%d"),
           "entries": sorted(table.values(), key=lambda e: e["key"])}
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description="measure per-shape launch choices into the table")
    ap.add_argument("--generate", action="store_true")
    ap.add_argument("--configs", default="1,2,3,4")
    ap.add_argument("--out", default=TABLE_PATH)
    ap.add_argument("--reps", type=int, default=20)
    a = ap.parse_args()
    if a.generate:
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        if root not in sys.path:
            sys.path.insert(0, root)
        generate([int(c) for c in a.configs.split(",")], a.out, a.reps)
