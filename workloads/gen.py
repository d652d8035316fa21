"""Seeded generators for the five synthetic multi-LoRA workloads.

The workloads stand in for the serving runs that vLLM PR #13096 ("[V1] LoRA -
Add triton kernels for V1", benchmark_throughput section) and vLLM PR #11613
("[Do Not Merge] - LoRA V1 Reference PR", Benchmarks section) measure on
ShareGPT prompts with Llama-2-7b-hf, 4 adapters at rank 8.  Neither the dataset,
the model nor the trained adapter is used here: request-length mixes are drawn
from a lognormal law, activations and adapter weights from scaled normals, and
the shapes are those of Llama-2-7B / 70B projections.

Recipe (fixed, so every consumer sees identical bits):

* ``rng = numpy.random.default_rng(seed)``; the draw order is: adapter map,
  then x, then A for each slice, then B for each slice, then y0.
* Normal draws are float32 (``rng.standard_normal(..., dtype=float32)``),
  multiplied by a float32 factor, then rounded to bfloat16 with
  round-to-nearest-even.  x ~ N(0,1); A_s ~ N(0,1)/sqrt(hidden);
  B_s ~ N(0,1)/sqrt(rank); y0 ~ N(0,1).
* Request lengths: ``max(1, round(exp(log(median) + sigma*z)))`` with
  sigma = 1.0 and z ~ N(0,1) drawn one request at a time until the lengths
  cover T; the last request is truncated so the total is exactly T.  A cap
  applies where the workload names one.  Each request then draws ``u`` (for the
  no-adapter probability) and an adapter id, in that order, even when ``u``
  makes the adapter unused.
* Zipf(s) is the finite law over ranks 1..L with P(k) proportional to k**-s;
  the adapter id is k-1.

bf16 values are carried as their raw uint16 bit patterns.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

# --------------------------------------------------------------------------
# The five workloads.  ``ids`` describes how the token -> adapter map is drawn.
# --------------------------------------------------------------------------
WORKLOADS = [
    dict(
        name="tiny",
        num_tokens=16, hidden=256, slices=[256], rank=8, max_loras=2, scale=1.0,
        ids=dict(kind="uniform", values=[-1, 0, 1]),
    ),
    dict(
        name="llama2_7b_qkv_decode",
        num_tokens=256, hidden=4096, slices=[4096, 4096, 4096], rank=8, max_loras=4,
        scale=2.0,
        ids=dict(kind="uniform", values=[0, 1, 2, 3]),
    ),
    dict(
        name="llama2_7b_gate_up_mixed_prefill",
        num_tokens=8192, hidden=4096, slices=[11008, 11008], rank=16, max_loras=4,
        scale=1.0,
        ids=dict(kind="requests", median=200.0, cap=2048, law="uniform", num_adapters=4,
                 p_none=0.2),
    ),
    dict(
        name="llama2_7b_down_proj",
        num_tokens=2048, hidden=11008, slices=[4096], rank=64, max_loras=16, scale=1.0,
        ids=dict(kind="zipf_iid", s=1.1, num_adapters=16),
    ),
    dict(
        name="llama2_70b_gqa_qkv",
        num_tokens=4096, hidden=8192, slices=[8192, 1024, 1024], rank=32, max_loras=64,
        scale=1.0,
        ids=dict(kind="requests", median=64.0, cap=None, law="zipf", s=1.0,
                 num_adapters=64, p_none=0.1),
    ),
]

LOGNORMAL_SIGMA = 1.0


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return raw bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input value")
    bits = a.view(np.uint32)
    # finite float32 patterns stay below 0xFF800000, so the sum cannot wrap
    out = bits >> 16
    out &= 1
    out += 0x7FFF
    out += bits
    out >>= 16
    return out.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    num_tokens: int
    max_tokens: int
    hidden: int
    slices: List[int]
    rank: int
    max_loras: int
    scale: float
    mapping: np.ndarray            # int32 [num_tokens]
    x: np.ndarray                  # uint16 (bf16 bits) [max_tokens, hidden]
    lora_a: List[np.ndarray]       # per slice: uint16 [max_loras, rank, hidden]
    lora_b: List[np.ndarray]       # per slice: uint16 [max_loras, n_s, rank]
    y0: np.ndarray                 # uint16 [max_tokens, n_total]

    @property
    def n_total(self) -> int:
        return int(sum(self.slices))

    @property
    def num_slices(self) -> int:
        return len(self.slices)


def _normal_bf16(rng, shape, factor) -> np.ndarray:
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if factor != 1.0:
        z *= np.float32(factor)
    return bf16_bits_from_f32(z)


def _zipf_probs(s: float, n: int) -> np.ndarray:
    k = np.arange(1, n + 1, dtype=np.float64)
    w = k ** (-s)
    return w / w.sum()


def _request_lengths(rng, total: int, median: float, cap: Optional[int]) -> List[int]:
    lengths = []
    covered = 0
    mu = math.log(median)
    while covered < total:
        z = float(rng.standard_normal())
        n = max(1, int(round(math.exp(mu + LOGNORMAL_SIGMA * z))))
        if cap is not None:
            n = min(n, cap)
        n = min(n, total - covered)
        lengths.append(n)
        covered += n
    return lengths


def _draw_mapping(rng, num_tokens: int, spec: dict) -> np.ndarray:
    kind = spec["kind"]
    if kind == "uniform":
        values = np.asarray(spec["values"], dtype=np.int32)
        idx = rng.integers(0, len(values), size=num_tokens)
        return values[idx].astype(np.int32)
    if kind == "zipf_iid":
        probs = _zipf_probs(spec["s"], spec["num_adapters"])
        return rng.choice(spec["num_adapters"], size=num_tokens, p=probs).astype(np.int32)
    if kind == "requests":
        lengths = _request_lengths(rng, num_tokens, spec["median"], spec.get("cap"))
        n_ad = spec["num_adapters"]
        probs = _zipf_probs(spec["s"], n_ad) if spec["law"] == "zipf" else None
        out = np.empty(num_tokens, dtype=np.int32)
        pos = 0
        for n in lengths:
            u = float(rng.random())
            if probs is None:
                ad = int(rng.integers(0, n_ad))
            else:
                ad = int(rng.choice(n_ad, p=probs))
            out[pos:pos + n] = -1 if u < spec["p_none"] else ad
            pos += n
        return out
    raise ValueError(f"unknown mapping kind {kind!r}")


def make_workload(index: int, seed: Optional[int] = None, num_tokens: Optional[int] = None,
                  max_tokens: Optional[int] = None) -> Workload:
    """Draw workload ``index`` (0..4) with ``seed`` (default: the index).

    ``num_tokens`` overrides the batch size (same shapes otherwise), used for
    reduced-size parity cases; ``max_tokens`` (default ``num_tokens``) sizes the
    row dimension of x and y0, rows beyond ``num_tokens`` being extra draws.
    """
    cfg = WORKLOADS[index]
    rng = np.random.default_rng(index if seed is None else seed)
    T = cfg["num_tokens"] if num_tokens is None else int(num_tokens)
    maxT = T if max_tokens is None else int(max_tokens)
    if maxT < T:
        raise ValueError("max_tokens < num_tokens")
    hidden, rank, L = cfg["hidden"], cfg["rank"], cfg["max_loras"]
    slices = list(cfg["slices"])
    mapping = _draw_mapping(rng, T, cfg["ids"])
    x = _normal_bf16(rng, (maxT, hidden), 1.0)
    lora_a = [_normal_bf16(rng, (L, rank, hidden), 1.0 / math.sqrt(hidden)) for _ in slices]
    lora_b = [_normal_bf16(rng, (L, n, rank), 1.0 / math.sqrt(rank)) for n in slices]
    y0 = _normal_bf16(rng, (maxT, sum(slices)), 1.0)
    return Workload(cfg["name"], T, maxT, hidden, slices, rank, L, float(cfg["scale"]),
                    mapping, x, lora_a, lora_b, y0)


def make_mapping(index: int, seed: Optional[int] = None,
                 num_tokens: Optional[int] = None) -> np.ndarray:
    """Only the adapter map of workload ``index`` (identical to the one
    ``make_workload`` draws with the same seed and size: it is the first draw)."""
    cfg = WORKLOADS[index]
    rng = np.random.default_rng(index if seed is None else seed)
    T = cfg["num_tokens"] if num_tokens is None else int(num_tokens)
    return _draw_mapping(rng, T, cfg["ids"])


def make_custom_workload(seed: int, num_tokens: int, hidden: int, slices: List[int], rank: int,
                         max_loras: int, scale: float, mapping: np.ndarray,
                         max_tokens: Optional[int] = None, name: str = "custom") -> Workload:
    """Normal-valued workload with an explicit adapter map (edge-case and fuzz tests)."""
    rng = np.random.default_rng(seed)
    maxT = num_tokens if max_tokens is None else int(max_tokens)
    mapping = np.asarray(mapping, dtype=np.int32).reshape(-1)
    assert mapping.shape[0] == num_tokens
    x = _normal_bf16(rng, (maxT, hidden), 1.0)
    lora_a = [_normal_bf16(rng, (max_loras, rank, hidden), 1.0 / math.sqrt(hidden))
              for _ in slices]
    lora_b = [_normal_bf16(rng, (max_loras, n, rank), 1.0 / math.sqrt(rank)) for n in slices]
    y0 = _normal_bf16(rng, (maxT, sum(slices)), 1.0)
    return Workload(name, num_tokens, maxT, hidden, list(slices), rank, max_loras, float(scale),
                    mapping, x, lora_a, lora_b, y0)


def make_integer_exact_workload(seed: int, num_tokens: int, hidden: int, slices: List[int],
                                rank: int, max_loras: int, scale: float = 1.0,
                                mapping: Optional[np.ndarray] = None,
                                nnz_per_row: int = 4) -> Workload:
    """Inputs whose every partial sum is a small integer.

    x and B are drawn from {-1, 0, 1}; each row of A holds at most
    ``nnz_per_row`` entries of +-1 (the rest zero); y0 holds integers in
    [-8, 8].  With scale in {0.5, 1, 2} every intermediate is exactly
    representable in float32, whatever the summation order.
    """
    rng = np.random.default_rng(seed)
    if mapping is None:
        mapping = rng.integers(-1, max_loras, size=num_tokens).astype(np.int32)
    mapping = np.asarray(mapping, dtype=np.int32)
    x = bf16_bits_from_f32(rng.integers(-1, 2, size=(num_tokens, hidden)).astype(np.float32))
    lora_a = []
    for _ in slices:
        a = np.zeros((max_loras, rank, hidden), dtype=np.float32)
        for li in range(max_loras):
            for k in range(rank):
                cols = rng.choice(hidden, size=min(nnz_per_row, hidden), replace=False)
                a[li, k, cols] = rng.choice(np.array([-1.0, 1.0], dtype=np.float32),
                                            size=cols.shape[0])
        lora_a.append(bf16_bits_from_f32(a))
    lora_b = [bf16_bits_from_f32(rng.integers(-1, 2, size=(max_loras, n, rank)).astype(np.float32))
              for n in slices]
    y0 = bf16_bits_from_f32(rng.integers(-8, 9, size=(num_tokens, sum(slices))).astype(np.float32))
    return Workload("integer_exact", num_tokens, num_tokens, hidden, list(slices), rank,
                    max_loras, float(scale), mapping, x, lora_a, lora_b, y0)


def make_fuzz_mapping(rng, num_tokens: int, max_loras: int, kind: str) -> np.ndarray:
    """Adapter maps for metadata fuzzing, including ids outside [-1, max_loras)."""
    if num_tokens == 0:
        return np.zeros(0, dtype=np.int32)
    if kind == "wild":
        return rng.integers(-5, max_loras + 5, size=num_tokens).astype(np.int32)
    if kind == "all_none":
        return np.full(num_tokens, -1, dtype=np.int32)
    if kind == "single":
        return np.full(num_tokens, int(rng.integers(0, max_loras)), dtype=np.int32)
    if kind == "runs":
        out = np.empty(num_tokens, dtype=np.int32)
        pos = 0
        while pos < num_tokens:
            n = int(rng.integers(1, 64))
            out[pos:pos + n] = int(rng.integers(-1, max_loras))
            pos += n
        return out
    if kind == "extreme":
        vals = np.array([np.iinfo(np.int32).min, np.iinfo(np.int32).max, -2, -1, 0,
                         max_loras - 1, max_loras], dtype=np.int32)
        return vals[rng.integers(0, len(vals), size=num_tokens)]
    raise ValueError(kind)


def workload_stats(w: Workload) -> dict:
    """Batch statistics and the algorithmic byte count of one step.

    Algorithmic bytes: x rows of tokens with an adapter; A and B of the adapters
    in use (every slice), once each; a read and a write of the y rows of tokens
    with an adapter; the adapter map and the sorted token order (4 bytes a token
    each).  Nothing is counted for tokens without an adapter.
    """
    ids = np.where((w.mapping >= -1) & (w.mapping < w.max_loras), w.mapping, -1)
    active = ids[ids >= 0]
    t_active = int(active.shape[0])
    uniq, counts = np.unique(active, return_counts=True)
    n_ad = int(uniq.shape[0])
    S, r, H, N = w.num_slices, w.rank, w.hidden, w.n_total
    x_bytes = t_active * H * 2
    a_bytes = n_ad * S * r * H * 2
    b_bytes = n_ad * N * r * 2
    y_bytes = 2 * t_active * N * 2
    idx_bytes = 2 * w.num_tokens * 4
    shrink_flops = 2 * t_active * S * r * H
    expand_flops = 2 * t_active * N * r
    return dict(
        num_tokens=w.num_tokens, active_tokens=t_active, active_adapters=n_ad,
        segment_min=int(counts.min()) if n_ad else 0,
        segment_median=float(np.median(counts)) if n_ad else 0.0,
        segment_max=int(counts.max()) if n_ad else 0,
        x_bytes=x_bytes, a_bytes=a_bytes, b_bytes=b_bytes, y_bytes=y_bytes,
        index_bytes=idx_bytes,
        shrink_bytes=x_bytes + a_bytes,
        expand_bytes=b_bytes + y_bytes,
        total_bytes=x_bytes + a_bytes + b_bytes + y_bytes + idx_bytes,
        shrink_flops=shrink_flops, expand_flops=expand_flops,
    )
