"""Schedules ("The task scheduler: mapping tasks to SMs": every wave order and placement
produces the same step): each named wave order, with round-robin and XCD placement, gives
bit-identical logits, residual stream, KV-cache writes, expert choices and activations;
the default schedule also matches the CPU reference.  Needs an MI355X."""
import numpy as np
import pytest

import decode_megakernel_amd as mkd
import synth
from parity import compare, gpu_step, oracle_step

pytestmark = pytest.mark.gpu

ORDERS = [mkd.ORDER_DEFAULT, mkd.ORDER_ATTN_FIRST, mkd.ORDER_MOE_FIRST, mkd.ORDER_INTERLEAVED]
PLACEMENTS = [mkd.PLACE_ROUND_ROBIN, mkd.PLACE_XCD]
FIELDS = ("logits", "hidden", "pool_after", "topk_ids", "topk_w", "route", "act", "q", "attn")


def _check_schedules(wl, name):
    ref = gpu_step(wl, schedule=(mkd.ORDER_DEFAULT, mkd.PLACE_ROUND_ROBIN))
    rep = compare(wl, ref, oracle_step(wl))
    print(f"[schedules] {name} default vs reference: hidden_rel={rep['hidden_rel']:.3g} "
          f"logits_rel={rep['logits_rel']:.3g}", flush=True)
    for order in ORDERS:
        for placement in PLACEMENTS:
            if (order, placement) == (mkd.ORDER_DEFAULT, mkd.PLACE_ROUND_ROBIN):
                continue
            print(f"[case] {name} order {order} placement {placement}", flush=True)
            g = gpu_step(wl, schedule=(order, placement))
            for f in FIELDS:
                a, b = getattr(g, f), getattr(ref, f)
                assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b), \
                    f"{name}: {f} differs between the default schedule and order {order} placement {placement}"


def test_schedules_tiny_ragged():
    _check_schedules(synth.ragged_workload(synth.TINY, [5, 64, 17, 0], spare_pages=3), "tiny-ragged")


def test_schedules_full_layer_8k_batch4():
    # batch 4 at 8K: the MoE-up claimers drain the shared queue (not the static split)
    _check_schedules(synth.layer_workload(ctx=8192, batch=4), "layer-8k-b4")
