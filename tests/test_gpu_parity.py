"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Metadata and integer-exact runs must match bit for bit; floating-point outputs
must meet max|y_gpu - y_ref| <= 1e-2 * rms(y_ref) + 1e-3 on top of the half
ulp of the bf16 output (the reading of the tolerance for a bf16 output), and
the shrink's fp32 projection the same bound without the rounding term.
"""

import numpy as np
import pytest
import torch

import oracle
import segmented_rank_gemm_amd as srg
from tests import gpu_harness as H
from workloads import (WORKLOADS, make_custom_workload, make_fuzz_mapping,
                       make_integer_exact_workload, make_mapping, make_workload)

pytestmark = pytest.mark.gpu

META_KEYS = H.META_KEYS
_sanitize = H.sanitize
_check_meta = H.check_meta
_full_check = H.full_check


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the GPU tests need a visible MI355X"
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), arch
    yield
    torch.cuda.synchronize()


def _run_metadata(mapping, T, max_tokens, L):
    meta = srg.LoraMeta(max_tokens, L)
    meta.sorted_token_ids.fill_(-7)
    for t in meta.tensors()[1:]:
        t.fill_(-99)
    m = torch.from_numpy(np.ascontiguousarray(mapping, dtype=np.int32)).cuda()
    srg.lora_prepare_metadata(m, T, meta)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in zip(META_KEYS, meta.tensors())}


# ------------------------------------------------------------------ metadata

@pytest.mark.parametrize("cfg", range(len(WORKLOADS)))
def test_metadata_bit_exact_full_size(cfg):
    mapping = make_mapping(cfg)
    T = mapping.shape[0]
    L = WORKLOADS[cfg]["max_loras"]
    got = _run_metadata(mapping, T, T + 37, L)
    _check_meta(got, oracle.prepare_metadata(mapping, L), T, T + 37, mapping=mapping, L=L)


FUZZ = [(0, 1, 1, "wild"), (0, 64, 8, "wild"), (1, 1, 1, "single"), (1, 5, 256, "wild"),
        (63, 64, 3, "runs"), (64, 64, 2, "wild"), (65, 100, 4, "extreme"), (1023, 1024, 16, "wild"),
        (1024, 1024, 64, "all_none"), (1025, 3000, 64, "runs"), (3000, 3000, 1, "wild"),
        (4096, 4096, 64, "wild"), (2049, 4096, 7, "extreme"),  # one full 512-thread block
        (4097, 5000, 256, "wild"), (8192, 8192, 4, "runs"), (20000, 20000, 256, "extreme"),
        (65536, 70000, 33, "wild"), (777, 777, 255, "single"),
        (1 << 20, (1 << 20) + 3, 256, "wild")]  # many blocks, every adapter slot


@pytest.mark.parametrize("T,maxT,L,kind", FUZZ)
def test_metadata_bit_exact_fuzz(T, maxT, L, kind):
    rng = np.random.default_rng(T * 7 + L)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    got = _run_metadata(mapping, T, maxT, L)
    _check_meta(got, oracle.prepare_metadata(mapping, L), T, maxT, mapping=mapping, L=L)


# --------------------------------------------------------- shrink + expand

REDUCED_T = [16, 200, 1000, 700, 900]


@pytest.mark.parametrize("cfg", range(len(WORKLOADS)))
@pytest.mark.parametrize("splits", ["default", 1, 3])
def test_step_parity_reduced(cfg, splits):
    w = make_workload(cfg, num_tokens=REDUCED_T[cfg], max_tokens=REDUCED_T[cfg] + 19)
    d = H.upload(w, num_splits=None if splits == "default" else splits, ldy_pad=8)
    H.run_step(d)
    torch.cuda.synchronize()
    _full_check(w, d)


@pytest.mark.parametrize("cfg", range(len(WORKLOADS)))
def test_step_parity_full_size(cfg):
    # full sizes, default number of parts: the launch configuration the benchmark times
    w = make_workload(cfg)
    d = H.upload(w)
    H.run_step(d)
    torch.cuda.synchronize()
    _full_check(w, d, literal=True)


@pytest.mark.parametrize("rank", [8, 16, 32, 64])
@pytest.mark.parametrize("splits", [1, 5])
@pytest.mark.parametrize("T", [300, 700])  # batches up to 512 tokens and larger take different kernels
def test_integer_exact_bitwise(rank, splits, T):
    w = make_integer_exact_workload(100 + rank, T, 328, [136, 40, 8], rank, 6,
                                    scale=2.0 if rank == 16 else 1.0)
    d = H.upload(w, num_splits=splits)
    H.run_step(d)
    torch.cuda.synchronize()
    ref = oracle.run_step(w)
    yg = H.from_dev_bf16(d.y)[:, :w.n_total]
    assert np.array_equal(yg, ref["y_bf16"])
    act = _sanitize(w.mapping, w.max_loras) >= 0
    assert np.array_equal(H.buf_sum(d)[:, act], ref["buf"][:, act])


SHAPES = [
    # (T, maxT, hidden, slices, rank, L, ldx_pad, ldy_pad, splits)
    (37, 40, 72, [8], 8, 1, 0, 0, 1),
    (130, 130, 264, [40, 136], 16, 3, 8, 16, 3),
    (257, 300, 1032, [128, 8, 24, 200], 32, 5, 0, 8, 64),
    (96, 96, 512, [64, 64, 64], 64, 2, 16, 0, 2),
    (500, 512, 2048, [1024], 64, 256, 0, 0, 4),
    (33, 33, 128, [16, 16, 16, 16], 8, 7, 0, 0, 7),
    # more than 512 token slots: the LDS-staged shrink, every output-group width
    (600, 640, 72, [8], 8, 1, 0, 0, 1),
    (700, 700, 264, [40, 136], 16, 3, 8, 16, 3),
    (600, 600, 200, [32, 32, 32], 16, 4, 0, 0, 1),
    (1030, 1100, 512, [64, 64, 64], 64, 2, 16, 0, 2),
    (900, 1024, 320, [64, 64, 64], 32, 9, 8, 8, 5),
    (777, 800, 1032, [128, 8, 24, 200], 32, 5, 0, 8, 64),
    (2000, 2048, 2048, [1024], 64, 256, 0, 0, 4),
    # extremes: one token slot; the widest hidden dimension; four rank-64 slices
    # (two output groups of eight blocks) in both shrink kernels
    (1, 1, 64, [8], 8, 1, 0, 0, 1),
    (40, 48, 65536, [64], 8, 2, 8, 0, 16),
    (600, 640, 65536, [16], 16, 3, 0, 8, 8),
    (300, 320, 384, [64, 32, 16, 8], 64, 3, 8, 8, 3),
    (700, 700, 384, [64, 32, 16, 8], 64, 3, 8, 8, 3),
    # every adapter slot in play with few tokens each: most tiles of the padded
    # order are single-token runs or gaps, and most of the walked tiles unused
    (100, 100, 256, [64, 64], 16, 256, 0, 0, 2),
    (300, 333, 512, [128], 8, 256, 8, 8, 5),
    (2000, 2040, 256, [96, 32], 16, 256, 0, 0, 3),
]


LARGE_BATCH_PARTS = [
    # (T, hidden, slices, rank, L, splits): batches of more than 512 tokens
    # (the LDS-staged shrink) on the down_proj, gate_up and 70B qkv shapes, from
    # two parts to the most parts the hidden dimension has 64-element chunks for
    (520, 11008, [4096], 64, 16, 2),
    (520, 11008, [4096], 64, 16, 64),
    (777, 1032, [256, 136], 64, 5, 5),    # rank 64 with 5 or 6 parts: the expand loads
    (5000, 2048, [1024], 64, 16, 6),      # every part in one batch; units over several rounds
    (1500, 4096, [2048, 2048], 16, 4, 8),
    (3000, 8192, [8192, 1024, 1024], 32, 64, 6),
    (2048, 1024, [512], 8, 1, 3),
    # 64 outputs (four blocks: four chunks in flight), parts of 35 chunks (a
    # three-chunk tail after the four-chunk groups), 41 chunks with the last
    # one partial (one-chunk tail) and 6 chunks (two-chunk tail)
    (600, 4480, [1024], 64, 8, 2),
    (700, 2600, [512, 256], 32, 5, 1),
    (640, 768, [128, 128, 128, 128], 16, 3, 2),
]


@pytest.mark.parametrize("T,hidden,slices,rank,L,splits", LARGE_BATCH_PARTS)
def test_large_batch_parts(T, hidden, slices, rank, L, splits):
    rng = np.random.default_rng(T + splits)
    mapping = rng.integers(-1, L, size=T)
    w = make_custom_workload(T, T, hidden, slices, rank, L, 1.0, mapping, max_tokens=T + 3)
    d = H.upload(w, num_splits=splits)
    H.run_step(d)
    torch.cuda.synchronize()
    _full_check(w, d)


def _large_fuzz_cases(n=16, seed=4099):
    """Seeded random shapes above 512 token slots (the LDS-staged shrink; the
    grid-strided and run-count walks of the rank-8/16 expand; the shared-B
    expand at ranks 32 and 64): token count, slots, hidden size, slices, rank,
    adapter slots, map kind, part count and row padding all drawn."""
    rng = np.random.default_rng(seed)
    kinds = ["wild", "runs", "extreme", "single", "all_none"]
    out = []
    for i in range(n):
        maxT = int(rng.integers(513, 2561))
        T = int(rng.integers(max(1, maxT - 300), maxT + 1))
        hidden = int(rng.choice([64, 200, 512, 1032, 2048]))
        rank = int(rng.choice([8, 16, 32, 64]))
        S = int(rng.integers(1, 5))
        slices = [8 * int(v) for v in rng.integers(1, 97, size=S)]
        L = int(rng.choice([1, 3, 8, 17, 64]))
        splits = int(rng.integers(1, min(16, max(1, hidden // 64)) + 1))
        ldx_pad, ldy_pad = 8 * int(rng.integers(0, 3)), 8 * int(rng.integers(0, 3))
        out.append((T, maxT, hidden, slices, rank, L, kinds[i % len(kinds)], splits,
                    ldx_pad, ldy_pad, i))
    return out


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,kind,splits,ldx_pad,ldy_pad,seed",
                         _large_fuzz_cases())
def test_large_batch_step_fuzz(T, maxT, hidden, slices, rank, L, kind, splits, ldx_pad, ldy_pad,
                               seed):
    """The whole step through the fused entry point (two launches here) and the
    expand, against the oracle, on seeded random large-batch shapes."""
    print(f"[large fuzz] seed={seed} T={T} maxT={maxT} hidden={hidden} slices={slices} "
          f"rank={rank} L={L} kind={kind} splits={splits}", flush=True)
    rng = np.random.default_rng(10_000 + seed)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    w = make_custom_workload(20_000 + seed, T, hidden, slices, rank, L, 0.75, mapping,
                             max_tokens=maxT)
    d = H.upload(w, num_splits=splits, ldx_pad=ldx_pad, ldy_pad=ldy_pad)
    H.run_step_fused(d)
    torch.cuda.synchronize()
    _full_check(w, d)


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,ldx_pad,ldy_pad,splits", SHAPES)
def test_shape_sweep(T, maxT, hidden, slices, rank, L, ldx_pad, ldy_pad, splits):
    rng = np.random.default_rng(T + hidden)
    mapping = rng.integers(-2, L + 1, size=T)
    w = make_custom_workload(T, T, hidden, slices, rank, L, 0.5, mapping, max_tokens=maxT)
    d = H.upload(w, num_splits=splits, ldx_pad=ldx_pad, ldy_pad=ldy_pad)
    H.run_step(d)
    torch.cuda.synchronize()
    _full_check(w, d)


def test_empty_parts_decode_shape():
    # 20 parts of 256 over hidden 4096: parts 16..19 hold no columns, and their
    # loads must stay inside x and A (both end exactly where the data ends).
    w = make_workload(1)
    d = H.upload(w, num_splits=20)
    H.run_step(d)
    torch.cuda.synchronize()
    _full_check(w, d)


@pytest.mark.parametrize("scale", [-1.5, 0.0])
@pytest.mark.parametrize("T", [200, 900])
def test_scale_values(scale, T):
    # a negative scale flips every product; zero leaves y exactly as it was
    rng = np.random.default_rng(int(T + 10 * scale))
    mapping = rng.integers(-1, 4, size=T)
    w = make_custom_workload(T + 3, T, 512, [96, 32], 16, 4, scale, mapping)
    d = H.upload(w, num_splits=3)
    H.run_step(d)
    torch.cuda.synchronize()
    _full_check(w, d)
    if scale == 0.0:
        assert np.array_equal(H.from_dev_bf16(d.y)[:T, :w.n_total], w.y0[:T])


@pytest.mark.parametrize("kind", ["empty", "all_none", "single", "one_token"])
def test_degenerate_batches(kind):
    T = {"empty": 0, "all_none": 50, "single": 80, "one_token": 1}[kind]
    mapping = {"empty": np.zeros(0), "all_none": np.full(50, -1), "single": np.full(80, 2),
               "one_token": np.array([1])}[kind]
    w = make_custom_workload(9, T, 256, [64, 32], 16, 3, 1.0, mapping, max_tokens=max(T, 1) + 5)
    d = H.upload(w, ldy_pad=8)
    H.run_step(d)
    torch.cuda.synchronize()
    yg = H.from_dev_bf16(d.y)
    if kind in ("empty", "all_none"):
        assert np.array_equal(yg[:, :w.n_total], w.y0[:w.max_tokens])
        assert int(d.meta.num_active.item()) == 0
    else:
        _full_check(w, d)


def test_inputs_never_written():
    w = make_workload(0, num_tokens=16, max_tokens=24)
    d = H.upload(w)
    before = [t.clone() for t in [d.mapping, d.x, *d.lora_a, *d.lora_b]]
    H.run_step(d)
    torch.cuda.synchronize()
    for a, b in zip(before, [d.mapping, d.x, *d.lora_a, *d.lora_b]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_binding_rejects_bad_views():
    """The binding refuses, before any launch, views the library would misread:
    a strided map, x narrower than hidden, a transposed y, empty weight lists,
    host tensors; the buffers it was given stay as they were."""
    w = make_workload(0, num_tokens=16, max_tokens=24)
    d = H.upload(w, buf_fill=1.5)
    y0 = d.y.clone()
    strided = torch.zeros(2 * w.num_tokens, dtype=torch.int32, device="cuda")[::2]
    with pytest.raises(ValueError, match="contiguous 1-D"):
        srg.lora_prepare_metadata(strided, w.num_tokens, d.meta)
    with pytest.raises(ValueError, match="contiguous 1-D"):
        srg.lora_prepare_and_shrink(strided, w.num_tokens, d.x, d.lora_a, 1.0, d.buf,
                                    d.num_splits, d.meta)
    narrow = d.x[:, : w.hidden - 8]
    with pytest.raises(ValueError, match=">=hidden"):
        srg.lora_shrink(narrow, d.lora_a, 1.0, d.buf, d.num_splits, d.meta)
    with pytest.raises(ValueError, match="at least one slice"):
        srg.lora_shrink(d.x, [], 1.0, d.buf, d.num_splits, d.meta)
    with pytest.raises(ValueError, match="at least one slice"):
        srg.lora_expand(d.buf, d.num_splits, [], d.y, d.meta)
    yt = torch.zeros((d.y.shape[1], d.y.shape[0]), dtype=torch.bfloat16, device="cuda").t()
    with pytest.raises(ValueError, match="unit column stride"):
        srg.lora_expand(d.buf, d.num_splits, d.lora_b, yt, d.meta)
    with pytest.raises(TypeError, match="device tensor"):
        srg.lora_prepare_metadata(d.mapping.cpu(), w.num_tokens, d.meta)
    torch.cuda.synchronize()
    assert torch.equal(d.y.view(torch.int16), y0.view(torch.int16))
    assert bool((d.buf == 1.5).all())


def test_bitwise_deterministic():
    w = make_workload(4, num_tokens=900)
    outs = []
    for _ in range(3):
        d = H.upload(w)
        H.run_step(d)
        torch.cuda.synchronize()
        outs.append((H.from_dev_bf16(d.y), d.buf.cpu().numpy().view(np.uint32)))
    for y, b in outs[1:]:
        assert np.array_equal(y, outs[0][0])
        assert np.array_equal(b, outs[0][1])


def test_token_permutation_permutes_rows():
    w = make_workload(3, num_tokens=300)
    d = H.upload(w)
    H.run_step(d)
    perm = np.random.default_rng(3).permutation(w.num_tokens)
    w2 = make_custom_workload(0, w.num_tokens, w.hidden, w.slices, w.rank, w.max_loras, w.scale,
                              w.mapping[perm])
    w2.x, w2.y0, w2.lora_a, w2.lora_b = w.x[perm], w.y0[perm], w.lora_a, w.lora_b
    d2 = H.upload(w2, num_splits=d.num_splits)
    H.run_step(d2)
    torch.cuda.synchronize()
    assert np.array_equal(H.from_dev_bf16(d2.y), H.from_dev_bf16(d.y)[perm])


@pytest.mark.parametrize("T,hidden,slices,rank,L", [
    (300, 1024, [512, 256, 256], 8, 4),      # up to 512 token slots: register shrink
    (900, 2048, [1024], 64, 16),             # LDS shrink, shared-B expand
    (1200, 1024, [2048, 2048], 16, 6),       # LDS shrink, position-tile expand
])
def test_graph_replays_new_batches(T, hidden, slices, rank, L):
    # One capture, then batches of the same size with new adapter maps and
    # activations copied into the captured buffers before each replay (static
    # buffers, as a graph-captured serving loop uses them): every replay must
    # match the oracle for its own batch, however many adapters it has.
    rng = np.random.default_rng(T + rank)
    kinds = [rng.integers(-1, L, size=T), np.full(T, L - 1), np.full(T, -1),
             np.sort(rng.integers(0, 2, size=T)), rng.integers(-3, L + 3, size=T)]
    batches = [make_custom_workload(T + i, T, hidden, slices, rank, L, 0.75, m)
               for i, m in enumerate(kinds)]
    d = H.upload(batches[0])
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        H.run_step(d, stream=torch.cuda.current_stream())
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
        _full_check(w, d)


def test_graph_replay_matches_eager():
    w = make_workload(1, num_tokens=256)
    d = H.upload(w)
    y0 = d.y.clone()
    H.run_step(d)
    torch.cuda.synchronize()
    eager = H.from_dev_bf16(d.y)

    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    d.y.copy_(y0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        H.run_step(d, stream=torch.cuda.current_stream())
    for _ in range(4):
        d.y.copy_(y0)          # eager reset between replays, outside the graph
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(H.from_dev_bf16(d.y), eager)


def test_tuned_splits_give_parity():
    """The tuner times each candidate on copies of the operands, leaves the
    caller's tensors untouched, and its choice passes the parity check."""
    from segmented_rank_gemm_amd.tuning import tune_shrink_splits
    mapping = np.random.default_rng(11).integers(-1, 4, size=600).astype(np.int32)
    w = make_custom_workload(7, 600, 1024, [512, 256], 16, 4, 1.25, mapping)
    d = H.upload(w)
    srg.lora_prepare_metadata(d.mapping, w.num_tokens, d.meta)
    y_before = d.y.clone()
    res = tune_shrink_splits(d.x, d.lora_a, d.lora_b, d.y, float(w.scale), d.meta,
                             candidates=[1, 2, 4], rotate_bytes=1 << 24, reps=3)
    torch.cuda.synchronize()
    assert set(res["us"]) == {1, 2, 4} and res["best"] in (1, 2, 4)
    assert all(t > 0 for t in res["us"].values())
    assert torch.equal(d.y.view(torch.int16), y_before.view(torch.int16))
    d2 = H.upload(w, num_splits=res["best"])
    H.run_step(d2)
    torch.cuda.synchronize()
    _full_check(w, d2)


# ------------------------------------------------ fused prepare + shrink ----

PREP_CASES = [  # T, maxT, hidden, slices, rank, L, kind, splits
    (0, 16, 256, [256], 8, 2, "wild", 1),
    (1, 1, 256, [256], 8, 1, "single", 1),
    (16, 16, 256, [256], 8, 2, "wild", 2),
    (100, 128, 512, [96, 32], 16, 8, "wild", 3),
    (200, 256, 1024, [256, 256], 8, 4, "all_none", 2),
    (300, 300, 1024, [512, 256], 32, 64, "runs", 5),               # > 16 slots: two launches
    (480, 512, 1024, [512, 256], 32, 16, "wild", 5),
    (511, 512, 256, [256, 256, 256, 256], 8, 3, "extreme", 1),
    (512, 512, 2048, [1024], 64, 256, "wild", 16),
    (512, 512, 2048, [1024], 64, 16, "extreme", 16),
    (512, 512, 1024, [256, 256, 256, 256], 64, 16, "runs", 4),  # 16 output blocks: 2 groups
    (700, 720, 1024, [512, 512], 16, 4, "wild", 3),             # larger: two launches
    (3000, 3500, 512, [256, 128], 32, 40, "runs", 4),           # 512-thread metadata
    # one chunk per wave, A rows straight into LDS:
    (96, 96, 1000, [128], 8, 16, "wild", 4),       # 8 output blocks; the last part's last chunk partial
    (64, 80, 96, [40], 8, 5, "wild", 1),           # 40 outputs in 4 blocks; waves 2-3 have no chunk
    (33, 48, 200, [64, 64], 16, 3, "runs", 1),     # 6 blocks; a chunk of 8 elements
]


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,kind,splits", PREP_CASES)
def test_prepare_and_shrink_matches_two_calls(T, maxT, hidden, slices, rank, L, kind, splits):
    """Metadata and parts from the fused call equal those of lora_prepare_metadata
    + lora_shrink bit for bit (buf compared as raw words, its NaN fill included)."""
    rng = np.random.default_rng(T * 31 + L)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    w = make_custom_workload(T + 5, T, hidden, slices, rank, L, 1.5, mapping, max_tokens=maxT)
    d1 = H.upload(w, num_splits=splits)
    d2 = H.upload(w, num_splits=splits)
    srg.lora_prepare_metadata(d1.mapping, T, d1.meta)
    srg.lora_shrink(d1.x, d1.lora_a, float(w.scale), d1.buf, splits, d1.meta)
    srg.lora_prepare_and_shrink(d2.mapping, T, d2.x, d2.lora_a, float(w.scale), d2.buf, splits,
                                d2.meta)
    torch.cuda.synchronize()
    m1, m2 = H.meta_host(d1), H.meta_host(d2)
    _check_meta(m2, oracle.prepare_metadata(mapping, L), T, maxT, mapping=mapping, L=L)
    nt = int(m1["num_tiles"][0])
    assert np.array_equal(m1["sorted_token_ids"], m2["sorted_token_ids"])
    for k in ["active_lora_ids", "num_tokens_per_lora", "lora_token_start", "num_active",
              "num_tiles", "num_runs"]:
        assert np.array_equal(m1[k], m2[k]), k
    assert np.array_equal(m1["tile_token_ids"][:16 * nt], m2["tile_token_ids"][:16 * nt])
    assert np.array_equal(m1["tile_lora"][:nt], m2["tile_lora"][:nt])
    assert np.array_equal(d1.buf.view(torch.int32).cpu().numpy(),
                          d2.buf.view(torch.int32).cpu().numpy())
    # and the fused call's own result, expanded, against the oracle
    _expand_and_check(w, d2)


def _expand_and_check(w, d):
    srg.lora_expand(d.buf, d.num_splits, d.lora_b, d.y, d.meta)
    torch.cuda.synchronize()
    if w.num_tokens == 0:
        assert np.array_equal(H.from_dev_bf16(d.y)[:, :w.n_total], w.y0[:w.max_tokens])
    else:
        _full_check(w, d)


def _fused_fuzz_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    kinds = ["wild", "all_none", "single", "runs", "extreme"]
    out = []
    for i in range(n):
        maxT = int(rng.integers(1, 513))
        T = int(rng.integers(0, maxT + 1))
        L = int(rng.integers(1, 17))
        rank = int(rng.choice([8, 16, 32, 64]))
        S = int(rng.integers(1, 5))
        slices = [8 * int(rng.integers(1, 65)) for _ in range(S)]
        hidden = 8 * int(rng.integers(1, 257))
        splits = int(rng.integers(1, 18))
        out.append((T, maxT, hidden, slices, rank, L, kinds[i % len(kinds)], splits, i))
    return out


@pytest.mark.parametrize("T,maxT,hidden,slices,rank,L,kind,splits,seed", _fused_fuzz_cases())
def test_prepare_and_shrink_fuzz(T, maxT, hidden, slices, rank, L, kind, splits, seed):
    """Random small shapes through the fused launch: metadata and every part of
    buf equal to the two calls', word for word."""
    rng = np.random.default_rng(seed + 500)
    mapping = make_fuzz_mapping(rng, T, L, kind)
    w = make_custom_workload(seed, T, hidden, slices, rank, L, 0.5, mapping, max_tokens=maxT)
    d1 = H.upload(w, num_splits=splits)
    d2 = H.upload(w, num_splits=splits)
    srg.lora_prepare_metadata(d1.mapping, T, d1.meta)
    srg.lora_shrink(d1.x, d1.lora_a, float(w.scale), d1.buf, splits, d1.meta)
    srg.lora_prepare_and_shrink(d2.mapping, T, d2.x, d2.lora_a, float(w.scale), d2.buf, splits,
                                d2.meta)
    torch.cuda.synchronize()
    m1, m2 = H.meta_host(d1), H.meta_host(d2)
    nt = int(m1["num_tiles"][0])
    assert np.array_equal(m1["sorted_token_ids"], m2["sorted_token_ids"])
    for k in ["active_lora_ids", "num_tokens_per_lora", "lora_token_start", "num_active",
              "num_tiles", "num_runs"]:
        assert np.array_equal(m1[k], m2[k]), k
    assert np.array_equal(m1["tile_token_ids"][:16 * nt], m2["tile_token_ids"][:16 * nt])
    assert np.array_equal(m1["tile_lora"][:nt], m2["tile_lora"][:nt])
    assert np.array_equal(d1.buf.view(torch.int32).cpu().numpy(),
                          d2.buf.view(torch.int32).cpu().numpy())
    # and the fused call's own result, expanded, against the oracle
    _expand_and_check(w, d2)


@pytest.mark.parametrize("cfg", [0, 1])
def test_fused_step_parity_full_size(cfg):
    # the launch configuration the benchmark times for the decode step
    w = make_workload(cfg)
    d = H.upload(w)
    H.run_step_fused(d)
    torch.cuda.synchronize()
    _full_check(w, d, literal=True)


def test_fused_graph_replays_new_batches():
    T, hidden, slices, rank, L = 256, 1024, [512, 256, 256], 8, 6
    rng = np.random.default_rng(99)
    kinds = [rng.integers(-1, L, size=T), np.full(T, L - 1), np.full(T, -1),
             np.sort(rng.integers(0, 2, size=T)), rng.integers(-3, L + 3, size=T)]
    batches = [make_custom_workload(T + i, T, hidden, slices, rank, L, 0.75, m)
               for i, m in enumerate(kinds)]
    d = H.upload(batches[0])
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        H.run_step_fused(d, stream=torch.cuda.current_stream())
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
        _full_check(w, d)
