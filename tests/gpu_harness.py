"""Helpers for the GPU tests: move a seeded workload onto the device, run the
HIP path through the binding, bring results back, and apply the comparison
criteria against the oracle."""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

import oracle
import segmented_rank_gemm_amd as srg
from workloads import f32_from_bf16_bits
from workloads.device import from_dev_bf16, to_dev_bf16  # noqa: F401


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(bits).astype(np.float64)


@dataclasses.dataclass
class DeviceWorkload:
    w: object
    mapping: torch.Tensor
    x: torch.Tensor
    lora_a: List[torch.Tensor]
    lora_b: List[torch.Tensor]
    y: torch.Tensor
    meta: srg.LoraMeta
    buf: torch.Tensor
    num_splits: int


def upload(w, num_splits: Optional[int] = None, ldx_pad: int = 0, ldy_pad: int = 0,
           buf_fill: float = float("nan"), sorted_fill: int = -7) -> DeviceWorkload:
    maxT = w.max_tokens
    mapping = torch.from_numpy(np.ascontiguousarray(w.mapping, dtype=np.int32)).cuda()
    x_host = np.zeros((maxT, w.hidden + ldx_pad), dtype=np.uint16)
    x_host[:, :w.hidden] = w.x[:maxT]
    x = to_dev_bf16(x_host)
    y_host = np.full((maxT, w.n_total + ldy_pad), 0x7FC1, dtype=np.uint16)  # sentinel NaN pad
    y_host[:, :w.n_total] = w.y0[:maxT]
    y = to_dev_bf16(y_host)
    lora_a = [to_dev_bf16(a) for a in w.lora_a]
    lora_b = [to_dev_bf16(b) for b in w.lora_b]
    if num_splits is None:
        num_splits = srg.lora_shrink_default_splits(w.hidden, maxT, w.max_loras, w.num_slices,
                                                    w.rank)
    meta = srg.LoraMeta(maxT, w.max_loras)
    meta.sorted_token_ids.fill_(sorted_fill)
    buf = torch.full((num_splits, w.num_slices, maxT, w.rank), buf_fill, dtype=torch.float32,
                     device="cuda")
    return DeviceWorkload(w, mapping, x, lora_a, lora_b, y, meta, buf, num_splits)


def run_step(d: DeviceWorkload, stream=None) -> None:
    srg.lora_prepare_metadata(d.mapping, d.w.num_tokens, d.meta, stream)
    srg.lora_shrink(d.x, d.lora_a, float(d.w.scale), d.buf, d.num_splits, d.meta, stream)
    srg.lora_expand(d.buf, d.num_splits, d.lora_b, d.y, d.meta, stream)


def run_step_fused(d: DeviceWorkload, stream=None) -> None:
    """The same step through lora_prepare_and_shrink (metadata and shrink in one
    call) and lora_expand."""
    srg.lora_prepare_and_shrink(d.mapping, d.w.num_tokens, d.x, d.lora_a, float(d.w.scale), d.buf,
                                d.num_splits, d.meta, stream)
    srg.lora_expand(d.buf, d.num_splits, d.lora_b, d.y, d.meta, stream)


def run_step_single(d: DeviceWorkload, workspace, stream=None, wait_polls=None) -> None:
    """The same step through lora_fused_step (one launch where the sizes allow)."""
    srg.lora_fused_step(d.mapping, d.w.num_tokens, d.x, d.lora_a, d.lora_b, float(d.w.scale),
                        d.buf, d.num_splits, d.y, d.meta, workspace, wait_polls=wait_polls,
                        stream=stream)


META_KEYS = ["sorted_token_ids", "active_lora_ids", "num_tokens_per_lora", "lora_token_start",
             "num_active", "tile_token_ids", "tile_lora", "num_tiles", "num_runs"]


def meta_host(d: DeviceWorkload) -> dict:
    return {k: v.cpu().numpy() for k, v in zip(META_KEYS, d.meta.tensors())}


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |v| (8 significant bits; 2^-133 below 2^-126)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(a)          # a = m * 2^e, m in [0.5, 1)
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def y_report(y_gpu_bits: np.ndarray, y64: np.ndarray, y_ref_bits: np.ndarray) -> dict:
    """Tolerance max|y_gpu - y_ref| <= 1e-2 rms(y_ref) + 1e-3, read on top of the
    half-ulp that rounding the output to bf16 costs (see the design notes)."""
    g = bf16_to_f64(y_gpu_bits)
    rms = float(np.sqrt(np.mean(y64 * y64))) if y64.size else 0.0
    tol = 1e-2 * rms + 1e-3
    err = np.abs(g - y64)
    excess = err - 0.5 * ulp_bf16(y64)
    ref_rne = bf16_to_f64(y_ref_bits)
    return dict(
        tol=tol, rms=rms,
        max_excess_over_half_ulp=float(excess.max()) if excess.size else 0.0,
        max_abs_err_vs_y64=float(err.max()) if err.size else 0.0,
        literal_over_tol_vs_y64=int(np.sum(err > tol)),
        literal_over_tol_vs_rne=int(np.sum(np.abs(g - ref_rne) > tol)),
        ulp_mismatch_vs_rne=int(np.sum(y_gpu_bits != y_ref_bits)),
        n=int(y64.size),
    )


def buf_sum(d: DeviceWorkload) -> np.ndarray:
    """Sum over the shrink's parts, in part order, in float64: [S, max_tokens, r]."""
    b = d.buf.cpu().numpy().astype(np.float64)
    return b.sum(axis=0)


def sanitize(mapping, L):
    m = np.asarray(mapping, dtype=np.int64)
    return np.where((m >= -1) & (m < L), m, -1)


def check_meta(meta_gpu, ref, T, max_tokens, sorted_fill=-7, mapping=None, L=None):
    assert np.array_equal(meta_gpu["sorted_token_ids"][:T], ref["sorted_token_ids"])
    assert np.all(meta_gpu["sorted_token_ids"][T:max_tokens] == sorted_fill)
    for k in META_KEYS[1:5]:
        assert np.array_equal(meta_gpu[k], ref[k]), k
    if mapping is not None:
        # the padded tiles, bit for bit below num_tiles
        tiles = oracle.prepare_tiles(mapping, L)
        nt = int(tiles["num_tiles"][0])
        assert int(meta_gpu["num_tiles"][0]) == nt
        assert np.array_equal(meta_gpu["tile_token_ids"][:nt * 16], tiles["tile_token_ids"])
        assert np.array_equal(meta_gpu["tile_lora"][:nt], tiles["tile_lora"])
        assert np.array_equal(meta_gpu["num_runs"], oracle.count_runs(mapping, L))


def full_check(w, d, literal=False):
    T = w.num_tokens
    ref = oracle.run_step(w)
    check_meta(meta_host(d), ref, T, w.max_tokens, mapping=w.mapping[:T], L=w.max_loras)
    ids = sanitize(w.mapping, w.max_loras)
    act = ids >= 0
    # shrink: sum of the parts against the fp64 projection (rows with an adapter)
    bs = buf_sum(d)[:, :T]
    if act.any():
        b64 = ref["buf"][:, act]
        brms = float(np.sqrt(np.mean(b64 * b64)))
        berr = float(np.max(np.abs(bs[:, act] - b64)))
        assert berr <= 1e-2 * brms + 1e-3, (berr, brms)
    # expand
    yg = from_dev_bf16(d.y)
    rep = y_report(yg[:T, :w.n_total], ref["y64"][:, :w.n_total],
                     ref["y_bf16"][:, :w.n_total])
    assert rep["max_excess_over_half_ulp"] <= rep["tol"], rep
    # rows without an adapter untouched, bit for bit; so are pad columns and rows >= T
    assert np.array_equal(yg[:T][~act, :w.n_total], w.y0[:T][~act])
    assert np.all(yg[:, w.n_total:] == 0x7FC1)
    if w.max_tokens > T:
        assert np.array_equal(yg[T:w.max_tokens, :w.n_total], w.y0[T:w.max_tokens])
    # buf rows of tokens without an adapter keep their fill (NaN), in every part
    braw = d.buf.cpu().numpy()
    assert np.all(np.isnan(braw[:, :, :T][:, :, ~act]))
    if literal:
        print(f"\n[{w.name}] T={T} tol={rep['tol']:.4g} max_excess={rep['max_excess_over_half_ulp']:.3g} "
              f"literal_over_tol(y64)={rep['literal_over_tol_vs_y64']} "
              f"literal_over_tol(rne)={rep['literal_over_tol_vs_rne']} "
              f"ulp_mismatch(rne)={rep['ulp_mismatch_vs_rne']}/{rep['n']}", flush=True)
    return rep
