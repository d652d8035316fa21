"""lora_fused_step_static (no allocation: counters in the library's own device
array) against lora_fused_step (counters in a caller workspace), through the C
ABI: two calls in a row on one GPU, the second on a smaller batch, each
compared with the workspace call on the same inputs (metadata, parts and y bit
for bit) and with the oracle."""

import numpy as np
import pytest
import torch

import segmented_rank_gemm_amd as srg
from tests import gpu_harness as H
from workloads import make_custom_workload, make_workload

pytestmark = pytest.mark.gpu


def _same_bits(a, b):
    ma, mb = H.meta_host(a), H.meta_host(b)
    for k in H.META_KEYS:
        if k in ("tile_token_ids", "tile_lora"):
            nt = int(ma["num_tiles"][0])
            n = 16 * nt if k == "tile_token_ids" else nt
            assert np.array_equal(ma[k][:n], mb[k][:n]), k
        else:
            assert np.array_equal(ma[k], mb[k]), k
    assert np.array_equal(a.buf.view(torch.int32).cpu().numpy(), b.buf.view(torch.int32).cpu().numpy())
    assert np.array_equal(H.from_dev_bf16(a.y), H.from_dev_bf16(b.y))


def _one(w):
    ws = srg.fused_step_workspace(w.max_tokens, w.max_loras, w.num_slices, w.rank)
    assert ws is not None, "the batch must take the one-launch path"
    d_ws, d_static = H.upload(w), H.upload(w)
    srg.lora_fused_step(d_ws.mapping, w.num_tokens, d_ws.x, d_ws.lora_a, d_ws.lora_b,
                        float(w.scale), d_ws.buf, d_ws.num_splits, d_ws.y, d_ws.meta, ws)
    srg.lora_fused_step_static(d_static.mapping, w.num_tokens, d_static.x, d_static.lora_a,
                               d_static.lora_b, float(w.scale), d_static.buf, d_static.num_splits,
                               d_static.y, d_static.meta)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    _same_bits(d_static, d_ws)
    H.full_check(w, d_static)


def test_static_counters_two_calls_second_smaller():
    assert torch.cuda.is_available()
    # the decode batch (256 token slots, 16 tiles), then a smaller one (100 of 128)
    _one(make_workload(1))
    mapping = np.random.default_rng(8).integers(-1, 3, size=100)
    _one(make_custom_workload(8, 100, 512, [256, 128], 16, 3, 0.5, mapping, max_tokens=128))


def test_static_counters_largest_batch_and_refusal():
    # the largest batch the array serves: 512 token slots
    mapping = np.random.default_rng(9).integers(-1, 4, size=500)
    _one(make_custom_workload(9, 500, 1024, [512, 512], 8, 4, 1.0, mapping, max_tokens=512))
    # a batch beyond the one-launch sizes takes the multi-launch path: no array needed
    w = make_custom_workload(10, 700, 512, [256], 8, 4, 1.0,
                             np.random.default_rng(10).integers(-1, 4, size=700))
    d = H.upload(w)
    srg.lora_fused_step_static(d.mapping, w.num_tokens, d.x, d.lora_a, d.lora_b, float(w.scale),
                               d.buf, d.num_splits, d.y, d.meta)
    torch.cuda.synchronize()
    H.full_check(w, d)
    # and with the batch-order shrink beside the metadata (no array either):
    # the same bits as the default multi-launch call
    d2 = H.upload(w)
    srg.lora_fused_step_static(d2.mapping, w.num_tokens, d2.x, d2.lora_a, d2.lora_b,
                               float(w.scale), d2.buf, d2.num_splits, d2.y, d2.meta,
                               batch_order_shrink=True)
    torch.cuda.synchronize()
    _same_bits(d2, d)
