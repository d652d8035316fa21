"""Parity of the one-launch step (lora_fused_step) and of multi-layer graphs
that share one metadata result, through the C ABI, against the CPU oracle.

The one-launch step must write the same metadata and the same shrink parts as
lora_prepare_and_shrink (bit for bit: the batch-order shrink splits the work
exactly as the grouped one does), y within the tolerance of the path, and
leave its workspace zero-filled; a step whose waits are cut to nothing (every
expand unit then computes its tile's parts itself) must give the same bits.
"""

import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_amd as srg
from tests import gpu_harness as H
from workloads import make_custom_workload, make_fuzz_mapping, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need a visible MI355X"
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), arch
    yield
    torch.cuda.synchronize()


def _workspace(w):
    return srg.fused_step_workspace(w.max_tokens, w.max_loras, w.num_slices, w.rank)


def _run_fused(d, ws, wait_polls=None, stream=None, start_delay_ns="table", part_sums=False,
               batch_order_shrink=False, y_delay_ns="table"):
    srg.lora_fused_step(d.mapping, d.w.num_tokens, d.x, d.lora_a, d.lora_b, float(d.w.scale),
                        d.buf, d.num_splits, d.y, d.meta, ws, wait_polls=wait_polls,
                        stream=stream, start_delay_ns=start_delay_ns, part_sums=part_sums,
                        batch_order_shrink=batch_order_shrink, y_delay_ns=y_delay_ns)


def _check_against_two_calls(w, d_step, d_two):
    """Metadata and parts equal to lora_prepare_and_shrink's, word for word."""
    m1, m2 = H.meta_host(d_two), H.meta_host(d_step)
    nt = int(m1["num_tiles"][0])
    assert np.array_equal(m1["sorted_token_ids"], m2["sorted_token_ids"])
    for k in ["active_lora_ids", "num_tokens_per_lora", "lora_token_start", "num_active",
              "num_tiles", "num_runs"]:
        assert np.array_equal(m1[k], m2[k]), k
    assert np.array_equal(m1["tile_token_ids"][:16 * nt], m2["tile_token_ids"][:16 * nt])
    assert np.array_equal(m1["tile_lora"][:nt], m2["tile_lora"][:nt])
    assert np.array_equal(d_two.buf.view(torch.int32).cpu().numpy(),
                          d_step.buf.view(torch.int32).cpu().numpy())


def _check_y(w, d):
    if w.num_tokens == 0:
        assert np.array_equal(H.from_dev_bf16(d.y)[:, :w.n_total], w.y0[:w.max_tokens])
        return None
    return H.full_check(w, d)


STEP_CASES = [  # T, maxT, hidden, slices, rank, L, kind, splits
    (0, 16, 256, [256], 8, 2, "wild", 1),
    (1, 1, 64, [8], 8, 1, "single", 1),
    (16, 16, 256, [256], 8, 2, "wild", 2),
    (100, 128, 512, [96, 32], 16, 4, "wild", 3),
    (200, 256, 8192, [1024], 8, 3, "all_none", 2),          # parts of 4096: two chunk sets
    (255, 256, 4096, [4096, 4096, 4096], 8, 4, "runs", 16),
    (300, 320, 1024, [512, 256, 256, 8], 8, 8, "extreme", 5),  # 8 slots, 256 outputs
    (333, 400, 1032, [136, 8, 24, 200], 8, 6, "wild", 7),    # 192 outputs: two groups
    (64, 64, 256, [256, 256, 256, 256], 16, 4, "single", 4),  # 256 outputs: two groups of 8
    (511, 512, 2048, [1024, 128], 16, 4, "runs", 8),
    (512, 512, 4096, [1024, 512, 512], 16, 4, "wild", 16),
    (400, 512, 640, [64], 8, 5, "wild", 64),                  # more parts than 64-chunks hold
    # outside the one-launch sizes: the same call takes the multi-launch path
    (700, 720, 1024, [512, 512], 16, 4, "wild", 3),
    (300, 300, 1024, [512], 32, 4, "runs", 2),
    (256, 256, 512, [256], 8, 16, "wild", 4),
]


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,kind,splits", STEP_CASES)
def test_fused_step_parity(T, maxT, hidden, slices, rank, L, kind, splits):
    print(f"[fused step] T={T} maxT={maxT} hidden={hidden} slices={slices} rank={rank} L={L} "
          f"kind={kind} splits={splits}", flush=True)
    rng = np.random.default_rng(T * 13 + L + rank)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    w = make_custom_workload(T + 11, T, hidden, slices, rank, L, 1.25, mapping, max_tokens=maxT)
    d_two = H.upload(w, num_splits=splits, ldy_pad=8)
    d_step = H.upload(w, num_splits=splits, ldy_pad=8)
    ws = _workspace(w)
    srg.lora_prepare_and_shrink(d_two.mapping, T, d_two.x, d_two.lora_a, float(w.scale), d_two.buf,
                                splits, d_two.meta)
    srg.lora_expand(d_two.buf, splits, d_two.lora_b, d_two.y, d_two.meta)
    _run_fused(d_step, ws)
    torch.cuda.synchronize()
    _check_against_two_calls(w, d_step, d_two)
    _check_y(w, d_step)
    if ws is not None:
        assert int(ws.count_nonzero()) == 0, "the workspace must come back zero-filled"


@pytest.mark.parametrize("cfg", [0, 1])
def test_fused_step_full_size(cfg):
    # the launch configuration the benchmark times
    w = make_workload(cfg)
    d = H.upload(w)
    ws = _workspace(w)
    assert ws is not None  # both take the one-launch path
    _run_fused(d, ws)
    torch.cuda.synchronize()
    H.full_check(w, d, literal=True)
    assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,splits", [
    (256, 256, 4096, [4096, 4096, 4096], 8, 4, 16),
    (333, 400, 1032, [136, 8, 24, 200], 8, 6, 7),
])
def test_fused_step_short_waits_same_bits(T, maxT, hidden, slices, rank, L, splits):
    """wait_polls of 1, 4 and 16: some expand units run out of polls and
    compute their tile's parts while the shrink units still write and count
    theirs.  Same metadata, parts and y, bit for bit, as the step that waits;
    the workspace is zero-filled after every call, and a call that waits on
    the same workspace afterwards gives the same bits again."""
    rng = np.random.default_rng(T + 7)
    mapping = rng.integers(-1, L, size=T)
    w = make_custom_workload(T + 11, T, hidden, slices, rank, L, 1.25, mapping, max_tokens=maxT)
    ws = _workspace(w)
    d_ref = H.upload(w, num_splits=splits)
    _run_fused(d_ref, ws)
    torch.cuda.synchronize()
    y_ref = H.from_dev_bf16(d_ref.y)
    for polls in (1, 4, 16, None):
        d = H.upload(w, num_splits=splits)
        _run_fused(d, ws, wait_polls=polls)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, polls
        _check_against_two_calls(w, d, d_ref)
        assert np.array_equal(y_ref, H.from_dev_bf16(d.y)), polls
    H.full_check(w, d_ref)


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,splits", [
    (256, 256, 4096, [4096, 4096, 4096], 8, 4, 16),
    (333, 400, 1032, [136, 8, 24, 200], 8, 6, 7),
    (200, 256, 8192, [1024], 8, 3, 2),
    (100, 128, 512, [96, 32], 16, 4, 3),
])
def test_fused_step_without_waits_same_bits(T, maxT, hidden, slices, rank, L, splits):
    """wait_polls = 0: no expand unit waits; each computes its tile's parts
    itself.  Same metadata, parts and y, bit for bit, as the step that waits."""
    rng = np.random.default_rng(T + hidden)
    mapping = rng.integers(-1, L, size=T)
    w = make_custom_workload(T, T, hidden, slices, rank, L, 0.75, mapping, max_tokens=maxT)
    d1, d2 = H.upload(w, num_splits=splits), H.upload(w, num_splits=splits)
    ws = _workspace(w)
    _run_fused(d1, ws)
    _run_fused(d2, ws, wait_polls=0)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    _check_against_two_calls(w, d2, d1)
    assert np.array_equal(H.from_dev_bf16(d1.y), H.from_dev_bf16(d2.y))
    H.full_check(w, d2)


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,splits", [
    (256, 256, 4096, [4096, 4096, 4096], 8, 4, 16),
    (77, 96, 640, [40, 264], 16, 4, 3),
])
def test_fused_step_start_delay_same_bits(T, maxT, hidden, slices, rank, L, splits):
    """The expand units' hold-offs change timing only: none, the library's
    defaults, long ones and y held back longer than B give the same bits, and
    the workspace ends zero-filled each time."""
    rng = np.random.default_rng(T * 7 + rank)
    mapping = rng.integers(-1, L, size=T)
    w = make_custom_workload(T, T, hidden, slices, rank, L, 0.75, mapping, max_tokens=maxT)
    ws = _workspace(w)
    runs = []
    for y_delay, delay in ((0, 0), (None, None), (800, 4000), (3000, 500)):
        d = H.upload(w, num_splits=splits)
        _run_fused(d, ws, start_delay_ns=delay, y_delay_ns=y_delay)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, (y_delay, delay)
        runs.append(d)
    for d in runs[1:]:
        _check_against_two_calls(w, d, runs[0])
        assert np.array_equal(H.from_dev_bf16(runs[0].y), H.from_dev_bf16(d.y))
    H.full_check(w, runs[0])


def test_fused_step_y_beyond_4gib():
    """y rows 8 MiB apart, so that the step's y spans more than 4 GiB: the
    one-launch kernel then stores y through 64-bit addresses instead of the
    32-bit offsets of its written-through stores.  Same criteria; the row
    padding keeps its sentinel."""
    T, hidden, slices, rank, L = 512, 256, [128, 136], 8, 4
    ldy = (1 << 22) + 64  # elements: T * ldy * 2 bytes > 4 GiB
    assert T * ldy * 2 >= 1 << 32
    assert srg.lora_fused_step_launches(T, L, len(slices), rank) == 1
    rng = np.random.default_rng(4242)
    mapping = rng.integers(-1, L, size=T)
    w = make_custom_workload(4242, T, hidden, slices, rank, L, 1.5, mapping)
    d = H.upload(w)
    big = torch.full((T, ldy), 0x7FC1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    big[:, :w.n_total] = d.y[:, :w.n_total]
    d.y = big
    ws = _workspace(w)
    _run_fused(d, ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    ref = oracle.run_step(w)
    act = H.sanitize(w.mapping, L) >= 0
    yg = H.from_dev_bf16(big[:, :w.n_total])
    rep = H.y_report(yg, ref["y64"], ref["y_bf16"])
    assert rep["max_excess_over_half_ulp"] <= rep["tol"], rep
    assert np.array_equal(yg[~act], w.y0[~act])
    for lo in (w.n_total, ldy - 64):
        assert np.all(H.from_dev_bf16(big[:, lo:lo + 64]) == 0x7FC1), lo
    del big, d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,scale,splits", [
    (900, 1024, 2048, [1024], 64, 16, 0.75, 6),             # down_proj-like: 6 parts in one batch
    (1000, 1000, 1536, [384, 128], 64, 9, 1.25, 5),         # rank 64, 5 parts in one batch
    (1500, 1536, 1024, [512, 128, 128], 32, 12, 1.0, 7),    # GQA qkv-like: 6 output blocks
    (700, 768, 1024, [256], 64, 5, -0.5, 4),                 # parts a whole batch; negative scale
    (640, 640, 768, [384, 64], 32, 8, 0.5, 8),               # rank 32: batches of 8
    (800, 1024, 1024, [256], 64, 6, 1.0, 1),                 # one part: no sums
    (1100, 1100, 2056, [136, 264], 32, 64, 1.0, 3),          # 64 adapter slots, odd sizes
])
def test_part_sums_same_bits(T, maxT, hidden, slices, rank, L, scale, splits):
    """Large rank-32/64 batches through lora_fused_step with part_sums: the
    shrink sums each row's parts for the expand (workspace counters and
    plane).  Same meta, parts and y, bit for bit, as lora_prepare_and_shrink +
    lora_expand (which sum the parts in the expand) and as the step without
    part sums; a second call on the used workspace gives the same bits again;
    y within the path's tolerance of the oracle."""
    rng = np.random.default_rng(T + rank)
    mapping = rng.integers(-1, L, size=T)
    w = make_custom_workload(T + 5, T, hidden, slices, rank, L, scale, mapping, max_tokens=maxT)
    ws = _workspace(w)
    assert ws is not None and ws.numel() > 0
    d_two = H.upload(w, num_splits=splits)
    H.run_step_fused(d_two)
    runs = []
    for sums in (True, True, False):
        d = H.upload(w, num_splits=splits)
        _run_fused(d, ws, part_sums=sums)
        torch.cuda.synchronize()
        runs.append(d)
    for d in runs:
        _check_against_two_calls(w, d, d_two)
        assert np.array_equal(H.from_dev_bf16(d_two.y), H.from_dev_bf16(d.y))
    H.full_check(w, runs[0])


def _runs_mapping(rng, T, L, median=64):
    """Request runs: consecutive tokens of one adapter (some of none)."""
    out, t = [], 0
    while t < T:
        n = int(min(T - t, max(1, rng.lognormal(np.log(median), 1.0))))
        out += [int(rng.integers(-1, L))] * n
        t += n
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,kind,splits,scale", [
    (8192, 8192, 4096, [11008, 11008], 16, 4, "runs", 2, 1.0),    # the gate_up prefill shape
    (4096, 4096, 8192, [8192, 1024, 1024], 32, 64, "runs", 7, 1.0),  # the 70B qkv shape
    (1000, 1536, 1032, [136, 264], 8, 6, "runs", 3, -0.5),        # ragged tail, unused slots
    (700, 700, 640, [256], 64, 16, "iid", 5, 1.0),                # a map drawn per token
    (777, 1024, 520, [96, 32], 16, 3, "runs", 12, 1.0),           # empty parts (12 x 64 > 520)
    (600, 600, 512, [128], 16, 4, "none", 2, 1.0),                # no token has an adapter
])
def test_batch_order_shrink_same_bits(T, maxT, hidden, slices, rank, L, kind, splits, scale):
    """Large batches through lora_fused_step with batch_order_shrink: the
    shrink in batch order beside the metadata workgroups, one launch.  Same
    meta, parts and y, bit for bit, as the metadata kernel then the grouped
    shrink (lora_prepare_and_shrink + lora_expand); y within the path's
    tolerance of the oracle."""
    rng = np.random.default_rng(T * 3 + L)
    if kind == "runs":
        mapping = _runs_mapping(rng, T, L)
    elif kind == "iid":
        mapping = rng.integers(-1, L, size=T)
    else:
        mapping = np.full(T, -1, dtype=np.int64)
    w = make_custom_workload(T + 11, T, hidden, slices, rank, L, scale, mapping, max_tokens=maxT)
    ws = _workspace(w)
    d_two = H.upload(w, num_splits=splits)
    H.run_step_fused(d_two)
    d = H.upload(w, num_splits=splits)
    _run_fused(d, ws, batch_order_shrink=True)
    torch.cuda.synchronize()
    _check_against_two_calls(w, d, d_two)
    assert np.array_equal(H.from_dev_bf16(d_two.y), H.from_dev_bf16(d.y))
    _check_y(w, d)


def _large_option_cases(n=14, seed=91):
    """Random large shapes for the batch-order shrink and the part sums."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        rank = int(rng.choice([8, 16, 32, 64]))
        maxT = int(rng.integers(513, 2049))
        T = int(rng.integers(1, maxT + 1))
        S = int(rng.integers(1, 4))
        slices = [8 * int(rng.integers(1, 129)) for _ in range(S)]
        hidden = 8 * int(rng.integers(1, 1025))
        L = int(rng.integers(1, 33))
        splits = int(rng.integers(1, 13))
        kind = ["runs", "iid", "mixed"][i % 3]
        out.append((T, maxT, hidden, slices, rank, L, kind, splits, i))
    return out


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,kind,splits,seed", _large_option_cases())
def test_large_batch_options_fuzz(T, maxT, hidden, slices, rank, L, kind, splits, seed):
    """lora_fused_step on random large shapes with each of its large-batch
    options (batch-order shrink; part sums where they apply): the same meta,
    parts and y, bit for bit, as lora_prepare_and_shrink + lora_expand, twice
    on the same workspace."""
    rng = np.random.default_rng(1000 + seed)
    if kind == "runs":
        mapping = _runs_mapping(rng, T, L, median=48)
    elif kind == "iid":
        mapping = rng.integers(-1, L, size=T)
    else:
        mapping = _runs_mapping(rng, T, L, median=8)
    w = make_custom_workload(2000 + seed, T, hidden, slices, rank, L, 0.5, mapping, max_tokens=maxT)
    ws = _workspace(w)
    d_two = H.upload(w, num_splits=splits)
    H.run_step_fused(d_two)
    y_ref = H.from_dev_bf16(d_two.y)
    for opts in (dict(batch_order_shrink=True), dict(part_sums=True),
                 dict(batch_order_shrink=True)):
        d = H.upload(w, num_splits=splits)
        _run_fused(d, ws, **opts)
        torch.cuda.synchronize()
        _check_against_two_calls(w, d, d_two)
        assert np.array_equal(y_ref, H.from_dev_bf16(d.y)), opts
    H.full_check(w, d_two)


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,splits,opts", [
    (700, 768, 1024, [512], 64, 6, 6, dict(part_sums=True)),                 # counters + plane
    (900, 1024, 520, [256, 128], 16, 4, 3, dict(batch_order_shrink=True)),   # metadata beside the shrink
])
def test_large_batch_options_graph_replays(T, maxT, hidden, slices, rank, L, splits, opts):
    """One capture of lora_fused_step with a large-batch option, replayed on
    new batches copied into the captured buffers, with eager work and
    synchronisations between the replays.  Every replay gives the meta, parts
    and y of lora_prepare_and_shrink + lora_expand on its own batch, bit for
    bit, and y within the path's tolerance of the oracle."""
    rng = np.random.default_rng(T + rank)
    kinds = [_runs_mapping(rng, T, L, median=48), rng.integers(-1, L, size=T),
             np.full(T, -1), rng.integers(-3, L + 3, size=T), np.full(T, L - 1),
             _runs_mapping(rng, T, L, median=8)]
    batches = [make_custom_workload(3000 + i, T, hidden, slices, rank, L, 0.75, m, max_tokens=maxT)
               for i, m in enumerate(kinds)]
    d = H.upload(batches[0], num_splits=splits)
    ws = _workspace(batches[0])
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        _run_fused(d, ws, stream=torch.cuda.current_stream(), **opts)
    for w in batches:
        fresh = H.upload(w, num_splits=splits)
        d.w = w
        d.mapping.copy_(fresh.mapping)
        d.x.copy_(fresh.x)
        d.y.copy_(fresh.y)
        for dst, src in zip(d.lora_a + d.lora_b, fresh.lora_a + fresh.lora_b):
            dst.copy_(src)
        d.buf.fill_(float("nan"))
        d.meta.sorted_token_ids.fill_(-7)
        d_two = H.upload(w, num_splits=splits)
        H.run_step_fused(d_two)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check_against_two_calls(w, d, d_two)
        assert np.array_equal(H.from_dev_bf16(d_two.y), H.from_dev_bf16(d.y))
        if int((np.asarray(w.mapping) >= 0).sum()) > 0:
            H.full_check(w, d)


def _fused_step_fuzz_cases(n=20, seed=77):
    rng = np.random.default_rng(seed)
    kinds = ["wild", "all_none", "single", "runs", "extreme"]
    out = []
    for i in range(n):
        rank = int(rng.choice([8, 16]))
        maxT = int(rng.integers(1, 513))
        T = int(rng.integers(0, maxT + 1))
        S = int(rng.integers(1, 5))
        L = int(rng.integers(1, (8 if rank == 8 else 4) + 1))
        while L * S * rank > 256:
            S -= 1
        slices = [8 * int(rng.integers(1, 97)) for _ in range(S)]
        hidden = 8 * int(rng.integers(1, 513))
        splits = int(rng.integers(1, 21))
        out.append((T, maxT, hidden, slices, rank, L, kinds[i % len(kinds)], splits, i))
    return out


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,kind,splits,seed", _fused_step_fuzz_cases())
def test_fused_step_fuzz(T, maxT, hidden, slices, rank, L, kind, splits, seed):
    print(f"[fused step fuzz] seed={seed} T={T} maxT={maxT} hidden={hidden} slices={slices} "
          f"rank={rank} L={L} kind={kind} splits={splits}", flush=True)
    rng = np.random.default_rng(seed + 900)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    w = make_custom_workload(seed + 40, T, hidden, slices, rank, L, 0.5, mapping, max_tokens=maxT)
    assert srg.lora_fused_step_workspace_bytes(maxT, L, len(slices), rank) > 0
    d_two = H.upload(w, num_splits=splits)
    d_step = H.upload(w, num_splits=splits)
    ws = _workspace(w)
    srg.lora_prepare_and_shrink(d_two.mapping, T, d_two.x, d_two.lora_a, float(w.scale), d_two.buf,
                                splits, d_two.meta)
    _run_fused(d_step, ws)
    torch.cuda.synchronize()
    _check_against_two_calls(w, d_step, d_two)
    _check_y(w, d_step)
    assert int(ws.count_nonzero()) == 0


def test_fused_step_graph_replays_new_batches():
    """One capture of lora_fused_step, replayed on new batches copied into the
    captured buffers; eager work and synchronisations between the replays.
    Every replay matches the oracle for its own batch and leaves the workspace
    zero-filled for the next."""
    T, hidden, slices, rank, L = 256, 1024, [512, 256, 256], 8, 4
    rng = np.random.default_rng(5)
    kinds = [rng.integers(-1, L, size=T), np.full(T, L - 1), np.full(T, -1),
             np.sort(rng.integers(0, 2, size=T)), rng.integers(-3, L + 3, size=T),
             rng.integers(0, L, size=T)]
    batches = [make_custom_workload(T + i, T, hidden, slices, rank, L, 0.75, m)
               for i, m in enumerate(kinds)]
    d = H.upload(batches[0])
    ws = _workspace(batches[0])
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        _run_fused(d, ws, stream=torch.cuda.current_stream())
    for w in batches:
        fresh = H.upload(w, num_splits=d.num_splits)
        d.w = w
        d.mapping.copy_(fresh.mapping)
        d.x.copy_(fresh.x)
        d.y.copy_(fresh.y)
        for dst, src in zip(d.lora_a + d.lora_b, fresh.lora_a + fresh.lora_b):
            dst.copy_(src)
        d.buf.fill_(float("nan"))
        d.meta.sorted_token_ids.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        H.full_check(w, d)
        assert int(ws.count_nonzero()) == 0


# ------------------------------------------------------------- layer stacks

LAYERS = 4


def _layer_stack(T, hidden, slices, rank, L, kinds_seed, fused_every_layer):
    """One batch through LAYERS layers with their own x, A, B and y on one
    metadata result, captured as one graph: the first layer groups the batch
    (lora_prepare_and_shrink, or lora_fused_step), the others reuse its
    grouping (lora_shrink + lora_expand, or lora_fused_step again)."""
    rng = np.random.default_rng(kinds_seed)
    mapping = rng.integers(-1, L, size=T)
    layers = [make_custom_workload(1000 + 17 * l + kinds_seed, T, hidden, slices, rank, L,
                                   0.5 + 0.25 * l, mapping) for l in range(LAYERS)]
    devs = [H.upload(w) for w in layers]
    meta = devs[0].meta
    ws = _workspace(layers[0])
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        cur = torch.cuda.current_stream()
        for l, (w, d) in enumerate(zip(layers, devs)):
            if fused_every_layer:
                srg.lora_fused_step(d.mapping, T, d.x, d.lora_a, d.lora_b, float(w.scale), d.buf,
                                    d.num_splits, d.y, meta, ws, stream=cur)
            elif l == 0:
                srg.lora_prepare_and_shrink(d.mapping, T, d.x, d.lora_a, float(w.scale), d.buf,
                                            d.num_splits, meta, cur)
                srg.lora_expand(d.buf, d.num_splits, d.lora_b, d.y, meta, cur)
            else:
                srg.lora_shrink(d.x, d.lora_a, float(w.scale), d.buf, d.num_splits, meta, cur)
                srg.lora_expand(d.buf, d.num_splits, d.lora_b, d.y, meta, cur)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for l, (w, d) in enumerate(zip(layers, devs)):
        d.meta = meta  # every layer's checks read the one grouping
        print(f"[layer stack] layer {l}", flush=True)
        H.full_check(w, d)
    if ws is not None:
        assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("fused_every_layer", [False, True])
def test_layer_stack_decode_shape(fused_every_layer):
    # the Llama-2-7B qkv decode shape: 256 tokens, 4096 -> 3 x 4096, rank 8, 4 slots
    _layer_stack(256, 4096, [4096, 4096, 4096], 8, 4, 3, fused_every_layer)


@pytest.mark.parametrize("T,hidden,slices,rank,L", [
    (1200, 2048, [1024, 512], 16, 6),   # above 512 token slots: LDS shrink, rank-16 expand
    (900, 2048, [1024], 64, 16),        # shared-B rank-64 expand
])
def test_layer_stack_large_batch(T, hidden, slices, rank, L):
    _layer_stack(T, hidden, slices, rank, L, T, False)
