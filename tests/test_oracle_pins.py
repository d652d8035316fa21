"""Pins of the CPU oracle against what the mathematics fixes.

The pages print no worked example and no kernel-level value, so the oracle is
pinned by: library routines (stable argsort, unique counts, dense float64
matmul), closed forms (rank-1 outer product), invariants (untouched rows,
permutation, linearity), an exact-rational brute force on tiny inputs, and an
integer-exact mode checked against integer arithmetic.  Each pin is chosen so a
plausible slip in the oracle (dropped scale, transposed operand, wrong slice
offset, unstable grouping, double rounding) fails at least one of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import bruteforce as bf
from workloads import (bf16_bits_from_f32, f32_from_bf16_bits, make_custom_workload,
                       make_fuzz_mapping, make_integer_exact_workload, make_workload)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(bits):
    return f32_from_bf16_bits(bits).astype(np.float64)


def _sanitize(mapping, max_loras):
    m = np.asarray(mapping, dtype=np.int64)
    return np.where((m >= -1) & (m < max_loras), m, -1)


# ---------------------------------------------------------------- rounding --

@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (-2.5, 0xC020),
    (1 + 2**-8, 0x3F80),               # tie between 1 and 1+2^-7: even (1.0) wins
    (1 + 3 * 2**-8, 0x3F82),           # tie between 1+2^-7 and 1+2^-6: even (1+2^-6) wins
    (1 + 2**-8 + 2**-40, 0x3F81),      # just above the tie: a float32 detour would say 0x3F80
    (2**-133, 0x0001),                 # smallest subnormal
    (2**-134, 0x0000),                 # half of it: tie, rounds to even zero
    (3 * 2**-135, 0x0001),
    (3.3895313892515355e38, 0x7F7F),   # largest finite
    (3.4e38, 0x7F80),                  # overflow to +inf
    (0.0, 0x0000),
])
def test_round_bf16_ieee_values(value, bits):
    assert oracle.round_bf16(value) == bits


def test_round_bf16_matches_exact_rational_rounding():
    rng = np.random.default_rng(1234)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                           # values one float64 ulp either side of bf16 midpoints
                           [float(np.nextafter(1 + 2**-8, 2)), float(np.nextafter(1 + 2**-8, 0))]])
    for v in vals:
        assert oracle.round_bf16(float(v)) == bf.fraction_to_bf16(Fraction(float(v))), v


def test_round_bf16_agrees_with_float32_path_on_float32_values():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(5000) * 100).astype(np.float32)
    ours = oracle.round_bf16_array(v.astype(np.float64))
    assert np.array_equal(ours, bf16_bits_from_f32(v))


# ---------------------------------------------------------------- metadata --

def test_metadata_worked_example():
    # ids after sanitising (7 is out of range for max_loras=3): [2,-1,0,2,1,-1,0,-1]
    # groups in ascending id, -1 first, tokens in index order:
    #   -1: 1,5,7   0: 2,6   1: 4   2: 0,3
    meta = oracle.prepare_metadata(np.array([2, -1, 0, 2, 1, -1, 0, 7]), max_loras=3)
    assert meta["sorted_token_ids"].tolist() == [1, 5, 7, 2, 6, 4, 0, 3]
    assert meta["active_lora_ids"].tolist() == [0, 1, 2]
    assert meta["num_tokens_per_lora"].tolist() == [2, 1, 2]
    assert meta["lora_token_start"].tolist() == [3, 5, 6]
    assert meta["num_active"].tolist() == [3]


def test_metadata_padding_slots():
    meta = oracle.prepare_metadata(np.array([3, 3, -1, 0, 3]), max_loras=6)
    assert meta["active_lora_ids"].tolist() == [0, 3, -1, -1, -1, -1]
    assert meta["num_tokens_per_lora"].tolist() == [1, 3, 0, 0, 0, 0]
    assert meta["lora_token_start"].tolist() == [1, 2, 5, 5, 5, 5]
    assert meta["num_active"].tolist() == [2]


def test_metadata_empty_batch():
    meta = oracle.prepare_metadata(np.zeros(0, dtype=np.int32), max_loras=4)
    assert meta["num_active"].tolist() == [0]
    assert meta["active_lora_ids"].tolist() == [-1] * 4
    assert meta["lora_token_start"].tolist() == [0] * 4


FUZZ_KINDS = ["wild", "all_none", "single", "runs", "extreme"]


@pytest.mark.parametrize("kind", FUZZ_KINDS)
@pytest.mark.parametrize("T,L", [(1, 1), (37, 3), (1000, 16), (4096, 64), (5000, 256)])
def test_metadata_matches_library_routines(kind, T, L):
    rng = np.random.default_rng(T * 1000 + L)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    meta = oracle.prepare_metadata(mapping, L)
    ids = _sanitize(mapping, L)
    # M1: the grouping is the library's stable argsort of the sanitised ids
    assert np.array_equal(meta["sorted_token_ids"], np.argsort(ids, kind="stable"))
    # M2: active ids and counts are numpy.unique of the ids >= 0; starts follow
    uniq, counts = np.unique(ids[ids >= 0], return_counts=True)
    na = int(meta["num_active"][0])
    assert na == uniq.shape[0]
    assert np.array_equal(meta["active_lora_ids"][:na], uniq)
    assert np.array_equal(meta["num_tokens_per_lora"][:na], counts)
    n_none = int(np.sum(ids == -1))
    starts = n_none + np.concatenate([[0], np.cumsum(counts)[:-1]]) if na else np.zeros(0)
    assert np.array_equal(meta["lora_token_start"][:na], starts)
    assert np.all(meta["active_lora_ids"][na:] == -1)
    assert np.all(meta["num_tokens_per_lora"][na:] == 0)
    assert np.all(meta["lora_token_start"][na:] == T)
    # M3: a permutation, ids non-decreasing along it, indices increasing within a group
    srt = meta["sorted_token_ids"]
    assert np.array_equal(np.sort(srt), np.arange(T))
    sid = ids[srt]
    assert np.all(np.diff(sid) >= 0)
    same = np.diff(sid) == 0
    assert np.all(np.diff(srt)[same] > 0)
    assert int(counts.sum()) + n_none == T


@pytest.mark.parametrize("seed", range(5))
def test_metadata_matches_selection_brute_force(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 9))
    mapping = make_fuzz_mapping(rng, int(rng.integers(1, 120)), L, FUZZ_KINDS[seed])
    meta = oracle.prepare_metadata(mapping, L)
    ref = bf.metadata(mapping, L)
    for k, v in ref.items():
        assert meta[k].tolist() == v, k


# ------------------------------------------------ runs in batch order -------

def test_runs_worked_examples():
    # by hand: [2, -1, 0, 2, 1, -1, 0, 7] with 3 slots reads 7 as -1, leaving
    # the runs {0}, {2}, {3}, {4}, {6}
    assert oracle.count_runs(np.array([2, -1, 0, 2, 1, -1, 0, 7]), 3).tolist() == [5]
    # 0 0 0 | 1 1 | (-1) | 1 1 | 0: the -1 splits the ones
    assert oracle.count_runs(np.array([0, 0, 0, 1, 1, -1, 1, 1, 0]), 2).tolist() == [4]
    assert oracle.count_runs(np.array([5, 5, 5]), 4).tolist() == [0]
    assert oracle.count_runs(np.zeros(0, dtype=np.int32), 4).tolist() == [0]


@pytest.mark.parametrize("kind", FUZZ_KINDS)
@pytest.mark.parametrize("T,L", [(1, 1), (37, 3), (1000, 16), (4096, 64)])
def test_runs_properties(kind, T, L):
    import itertools
    rng = np.random.default_rng(T * 7 + L)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    ids = _sanitize(mapping, L)
    n = int(oracle.count_runs(mapping, L)[0])
    # the library's run-length grouping, keeping the groups of an adapter
    assert n == sum(1 for k, _ in itertools.groupby(ids.tolist()) if k >= 0)
    # bounds: at least one run per adapter present, at most one per token
    assert len(set(ids[ids >= 0].tolist())) <= n <= int(np.sum(ids >= 0))
    # a grouped batch (the stable sort of itself) has exactly one run per adapter
    assert int(oracle.count_runs(np.sort(ids), L)[0]) == len(set(ids[ids >= 0].tolist()))
    # splitting the batch: the halves' runs add up, less one where a run straddles the cut
    c = T // 2
    a, b = ids[:c], ids[c:]
    join = 1 if c > 0 and c < T and a[-1] >= 0 and a[-1] == b[0] else 0
    assert n == int(oracle.count_runs(a, L)[0]) + int(oracle.count_runs(b, L)[0]) - join


# ------------------------------------------------ padded tiles of the order --

def test_tiles_worked_example():
    # adapters 0 (tokens 2, 6), 1 (token 4), 2 (tokens 0, 3); S = 0, 2, 3 and
    # k = 0, 1, 2 give starts round_up(S + 15k, 16) = 0, 32, 48 by hand, so
    # tile 1 is the empty gap between adapters 0 and 1
    t = oracle.prepare_tiles(np.array([2, -1, 0, 2, 1, -1, 0, 7]), 3)
    want = np.full(64, -1)
    want[[0, 1, 32, 48, 49]] = [2, 6, 4, 0, 3]
    assert t["tile_token_ids"].tolist() == want.tolist()
    assert t["tile_lora"].tolist() == [0, -1, 1, 2]
    assert t["num_tiles"].tolist() == [4]


def test_tiles_empty_and_no_adapter():
    for mapping in (np.zeros(0, dtype=np.int32), np.full(40, -1)):
        t = oracle.prepare_tiles(mapping, 4)
        assert t["num_tiles"].tolist() == [0]
        assert t["tile_token_ids"].size == 0 and t["tile_lora"].size == 0


@pytest.mark.parametrize("kind", FUZZ_KINDS)
@pytest.mark.parametrize("T,L", [(1, 1), (37, 3), (1000, 16), (4096, 64), (5000, 256)])
def test_tiles_are_the_grouping_padded(kind, T, L):
    rng = np.random.default_rng(T * 1000 + L + 7)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    ids = _sanitize(mapping, L)
    t = oracle.prepare_tiles(mapping, L)
    tok, lora, nt = t["tile_token_ids"], t["tile_lora"], int(t["num_tiles"][0])
    assert tok.shape == (nt * 16,) and lora.shape == (nt,)
    # without the -1 entries: the tokens that have an adapter, in the library's
    # stable argsort order
    order = np.argsort(ids, kind="stable")
    assert np.array_equal(tok[tok >= 0], order[ids[order] >= 0])
    # every tile holds one adapter's tokens (or none, with adapter -1)
    tiles = tok.reshape(nt, 16)
    for m in range(nt):
        members = tiles[m][tiles[m] >= 0]
        if lora[m] < 0:
            assert members.size == 0
        else:
            assert members.size > 0 and np.all(ids[members] == lora[m])
    # each adapter's run starts at round_up(S_k + 15 k, 16) and is contiguous
    uniq, counts = np.unique(ids[ids >= 0], return_counts=True)
    s = 0
    for k, (l, c) in enumerate(zip(uniq, counts)):
        p = -(-(s + 15 * k) // 16) * 16
        assert np.all(ids[tok[p:p + c]] == l) and np.all(np.diff(tok[p:p + c]) > 0)
        s += c
    assert nt <= -(-T // 16) + L + 1
    if nt:
        assert lora[-1] >= 0  # no trailing empty tile


# ------------------------------------------------------- shrink and expand --

def _dense_reference(w, rows, lid, scale):
    """y0 + scale * (x A^T) B^T for the given rows, one adapter, numpy float64 matmul."""
    X = _f64(w.x[rows])
    out = _f64(w.y0[rows]).copy()
    off = 0
    for s, n in enumerate(w.slices):
        A = _f64(w.lora_a[s][lid])          # [r, hidden]
        B = _f64(w.lora_b[s][lid])          # [n, r]
        out[:, off:off + n] += (scale * (X @ A.T)) @ B.T
        off += n
    return out


def _small(seed, T=24, hidden=72, slices=(40, 16, 24), rank=8, L=3, scale=1.5, mapping=None):
    rng = np.random.default_rng(seed)
    if mapping is None:
        mapping = rng.integers(-1, L, size=T)
    return make_custom_workload(seed, T, hidden, list(slices), rank, L, scale, mapping)


def test_single_adapter_equals_dense_product():
    # P2: one adapter for the whole batch is a plain dense low-rank product
    w = _small(11, mapping=np.full(24, 2))
    out = oracle.run_step(w)
    ref = _dense_reference(w, np.arange(w.num_tokens), 2, float(np.float32(w.scale)))
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-12, atol=1e-12)


def test_per_adapter_dense_loop_equals_oracle():
    # P2: N small dense products, one per adapter (the "launch N small kernels"
    # correctness baseline of the MLC-LLM issue's Overview), match a mixed batch
    w = _small(12, T=60, rank=16, L=4)
    out = oracle.run_step(w)
    ids = _sanitize(w.mapping, w.max_loras)
    ref = _f64(w.y0[:w.num_tokens]).copy()
    for lid in range(w.max_loras):
        rows = np.nonzero(ids == lid)[0]
        if rows.size:
            ref[rows] = _dense_reference(w, rows, lid, float(np.float32(w.scale)))
    np.testing.assert_allclose(out["y64"], ref, rtol=1e-12, atol=1e-12)
    # buf too: per-slice dense x A^T
    for s in range(w.num_slices):
        for lid in range(w.max_loras):
            rows = np.nonzero(ids == lid)[0]
            if rows.size:
                want = float(np.float32(w.scale)) * (_f64(w.x[rows]) @ _f64(w.lora_a[s][lid]).T)
                np.testing.assert_allclose(out["buf"][s, rows], want, rtol=1e-12, atol=1e-12)


def test_rows_without_adapter_are_untouched():
    # P1
    w = _small(13, T=40)
    out = oracle.run_step(w)
    none = _sanitize(w.mapping, w.max_loras) < 0
    assert none.any()
    assert np.array_equal(out["y_bf16"][none], w.y0[:w.num_tokens][none])
    assert np.array_equal(out["y64"][none], _f64(w.y0[:w.num_tokens][none]))


def test_token_permutation_permutes_outputs():
    # P3
    w = _small(14, T=33)
    out = oracle.run_step(w)
    perm = np.random.default_rng(5).permutation(w.num_tokens)
    w2 = make_custom_workload(14, w.num_tokens, w.hidden, w.slices, w.rank, w.max_loras,
                              w.scale, w.mapping[perm])
    w2.x = w.x[perm]
    w2.y0 = w.y0[perm]
    w2.lora_a, w2.lora_b = w.lora_a, w.lora_b
    out2 = oracle.run_step(w2)
    assert np.array_equal(out2["y_bf16"], out["y_bf16"][perm])
    assert np.array_equal(out2["y64"], out["y64"][perm])


def test_rank_one_closed_form():
    # P4: rank 1 is an outer product: y = y0 + scale * (x . a) * b
    w = _small(15, T=20, rank=1, slices=(24, 8))
    out = oracle.run_step(w)
    ids = _sanitize(w.mapping, w.max_loras)
    sc = float(np.float32(w.scale))
    for t in range(w.num_tokens):
        off = 0
        for s, n in enumerate(w.slices):
            if ids[t] < 0:
                assert np.array_equal(out["y64"][t, off:off + n], _f64(w.y0[t, off:off + n]))
            else:
                xa = math.fsum(_f64(w.x[t]) * _f64(w.lora_a[s][ids[t], 0]))
                want = _f64(w.y0[t, off:off + n]) + (sc * xa) * _f64(w.lora_b[s][ids[t], :, 0])
                np.testing.assert_allclose(out["y64"][t, off:off + n], want, rtol=1e-13,
                                           atol=1e-13)
            off += n


def test_exact_rational_brute_force_tiny():
    # P5: dyadic inputs make the exact result computable
    w = _small(16, T=6, hidden=16, slices=(8, 8), rank=2, L=2, scale=0.75)
    out = oracle.run_step(w)
    buf, y = bf.lora_exact(w.mapping, w.x, w.lora_a, w.lora_b, w.y0[:w.num_tokens],
                           w.max_loras, w.rank, float(np.float32(w.scale)))
    for t in range(w.num_tokens):
        for c in range(w.n_total):
            ex = y[t][c]
            assert abs(out["y64"][t, c] - float(ex)) <= 1e-12 * max(1.0, abs(float(ex)))
            assert out["y_bf16"][t, c] == bf.fraction_to_bf16(ex)
        for s in range(w.num_slices):
            if buf[s][t] is not None:
                for k in range(w.rank):
                    assert abs(out["buf"][s, t, k] - float(buf[s][t][k])) <= 1e-13


def test_linearity_zero_weights_slices_and_batch_split():
    # P6
    w = _small(17, T=30)
    base = oracle.run_step(w)
    ids = _sanitize(w.mapping, w.max_loras)
    act = ids >= 0
    # scale is applied once: doubling it doubles buf exactly and the delta to 1e-12
    w2 = _small(17, T=30, scale=3.0)
    dbl = oracle.run_step(w2)
    assert np.array_equal(dbl["buf"][:, act], 2.0 * base["buf"][:, act])
    y0 = _f64(w.y0[:w.num_tokens])
    np.testing.assert_allclose(dbl["y64"] - y0, 2.0 * (base["y64"] - y0), rtol=1e-12, atol=1e-12)
    # zero adapter weights leave y as it was
    wz = _small(17, T=30)
    wz.lora_b = [np.zeros_like(b) for b in wz.lora_b]
    z = oracle.run_step(wz)
    assert np.array_equal(z["y_bf16"], wz.y0[:wz.num_tokens])
    # each slice on its own gives the same columns
    off = 0
    for s, n in enumerate(w.slices):
        ws = make_custom_workload(17, w.num_tokens, w.hidden, [n], w.rank, w.max_loras,
                                  w.scale, w.mapping)
        ws.x, ws.lora_a, ws.lora_b = w.x, [w.lora_a[s]], [w.lora_b[s]]
        ws.y0 = np.ascontiguousarray(w.y0[:, off:off + n])
        one = oracle.run_step(ws)
        assert np.array_equal(one["y64"], base["y64"][:, off:off + n])
        off += n
    # two half batches give the same rows
    h = w.num_tokens // 2
    for lo, hi in [(0, h), (h, w.num_tokens)]:
        wh = make_custom_workload(17, hi - lo, w.hidden, w.slices, w.rank, w.max_loras, w.scale,
                                  w.mapping[lo:hi])
        wh.x, wh.y0 = w.x[lo:hi], w.y0[lo:hi]
        wh.lora_a, wh.lora_b = w.lora_a, w.lora_b
        part = oracle.run_step(wh)
        assert np.array_equal(part["y64"], base["y64"][lo:hi])


@pytest.mark.parametrize("rank,scale", [(8, 1.0), (64, 2.0), (16, 0.5)])
def test_integer_exact_mode_matches_integer_arithmetic(rank, scale):
    # P7: every partial sum is an integer (or a half-integer for scale 0.5), so
    # fp64 is exact; compare with int64 arithmetic done independently
    w = make_integer_exact_workload(21 + rank, 48, 96, [40, 24], rank, 5, scale)
    out = oracle.run_step(w)
    ids = _sanitize(w.mapping, w.max_loras)
    X = _f64(w.x).astype(np.int64)
    Y0 = _f64(w.y0).astype(np.int64)
    num = int(round(scale * 2))  # scale = num / 2
    for t in range(w.num_tokens):
        want = Y0[t].astype(object) * 2
        if ids[t] >= 0:
            off = 0
            for s, n in enumerate(w.slices):
                A = _f64(w.lora_a[s][ids[t]]).astype(np.int64)
                B = _f64(w.lora_b[s][ids[t]]).astype(np.int64)
                bufv = (A @ X[t]) * num          # 2 * buf, integer
                want[off:off + n] = want[off:off + n] + B @ bufv
                off += n
        got2 = out["y64"][t] * 2
        assert np.array_equal(got2, want.astype(np.float64)), t
        for c in range(w.n_total):
            assert out["y_bf16"][t, c] == bf.fraction_to_bf16(Fraction(int(want[c]), 2))


def test_out_of_range_ids_count_as_no_adapter():
    w = _small(31, T=16, mapping=np.array([0, 5, -2, 1, 2, 99, -1, 0, 1, 2, 3, -7, 0, 0, 1, 2]))
    out = oracle.run_step(w)
    w2 = _small(31, T=16, mapping=_sanitize(w.mapping, w.max_loras))
    out2 = oracle.run_step(w2)
    for k in ("sorted_token_ids", "active_lora_ids", "num_tokens_per_lora", "y_bf16"):
        assert np.array_equal(out[k], out2[k]), k


def test_golden_tiny_exact_values():
    with open(os.path.join(GOLDEN, "tiny_exact.json")) as f:
        g = json.load(f)
    w = _small(g["seed"], T=g["num_tokens"], hidden=g["hidden"], slices=tuple(g["slices"]),
               rank=g["rank"], L=g["max_loras"], scale=g["scale"],
               mapping=np.array(g["mapping"]))
    out = oracle.run_step(w)
    assert out["sorted_token_ids"].tolist() == g["sorted_token_ids"]
    for t, row in enumerate(g["y_exact"]):
        for c, s in enumerate(row):
            ex = Fraction(s)
            assert abs(out["y64"][t, c] - float(ex)) <= 1e-12 * max(1.0, abs(float(ex)))
    assert out["y_bf16"].tolist() == g["y_bf16"]


def test_config_shapes():
    w = make_workload(0)
    assert (w.num_tokens, w.hidden, w.slices, w.rank, w.max_loras) == (16, 256, [256], 8, 2)
    assert set(np.unique(w.mapping).tolist()) <= {-1, 0, 1}
