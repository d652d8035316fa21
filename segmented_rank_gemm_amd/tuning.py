"""Per-shape choice of the shrink's hidden-dimension parts, by measurement.

vLLM PR #11613 "[Do Not Merge] - LoRA V1 Reference PR" lists autotuning the V1
LoRA kernels among the follow-up items of its split plan.  The one free launch
parameter of the shrink + expand pair here is ``num_splits``: the number of
contiguous hidden-dimension parts the shrink computes separately and the
expand sums.  More parts spread a batch over more workgroups; fewer parts mean
fewer partial rows for the expand to read and less start-up per unit.  Where
the optimum lies depends on how the batch's tiles round against the compute
units, and the tile count is a property of the batch's adapter mix, known only
once the batch is grouped.  ``lora_shrink_default_splits`` is a rule on the
sizes alone; ``tune_shrink_splits`` settles the question for a representative
batch by timing the pair for each candidate and returning the fastest, to be
stored with the shape (``num_splits`` fixes the ``buf`` shape, so a captured
graph keeps the value it was captured with).

This is a host-side utility for an offline tuning step, not part of the path:
it only calls the library's entry points, allocates its own copies of the
operands with torch, synchronises, and never writes the caller's tensors.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence

import torch

from . import (LORA_MAX_SPLITS, LoraMeta, lora_expand, lora_shrink,
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
            lora_expand(bufs[i], n, o["b"], o["y"], meta, stream)

        for i in range(copies):  # eager pass first (and a check that the launch is accepted)
            pair(i, None)
        torch.cuda.synchronize()
        us[n] = _graph_seconds(pair, copies, reps) * 1e6
        del bufs
    del ops
    torch.cuda.synchronize()
    best = min(us, key=us.get)
    return {"best": best, "default": default, "us": us}
