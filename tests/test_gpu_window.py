"""GPU parity of local-attention layers (layers that attend to the last W positions;
the page's section "Tasks" runs the attention drain "only for full-attention layers"):
one decode step through the C-ABI against the CPU reference, with windows that start
mid-page, on a page boundary and before the first position.  Needs an MI355X."""
import dataclasses

import pytest

import synth
from parity import compare, gpu_step, oracle_step

pytestmark = pytest.mark.gpu


def _report(name, rep):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                          for k, v in rep.items()), flush=True)


@pytest.mark.parametrize("window,full_every,seq_lens", [
    (21, 2, [5, 64, 17, 0]),      # layer 0 local (window from mid-page), layer 1 full
    (21, 2, [33, 1, 100]),
    (16, 3, [47, 31]),            # window starting on a page boundary; both layers local
    (1, 3, [20, 9]),              # the new token only
])
def test_tiny_local_layers(window, full_every, seq_lens):
    geom = dataclasses.replace(synth.TINY, attn_window=window, full_every=full_every)
    wl = synth.ragged_workload(geom, seq_lens, spare_pages=3)
    print(f"[case] tiny local window={window} full_every={full_every} {seq_lens}", flush=True)
    g = gpu_step(wl, mode=0)
    r = oracle_step(wl)
    _report(f"tiny-local-{window}-{full_every}-{seq_lens}", compare(wl, g, r))


def test_full_layer_8k_local():
    geom = dataclasses.replace(synth.LAYER, attn_window=4000, full_every=2)
    wl = synth.make_workload("layer-local-b1-ctx8192", geom, [8192], spare_pages=8)
    print("[case] full-size local layer b1 ctx8192 window 4000", flush=True)
    g = gpu_step(wl, mode=0)
    r = oracle_step(wl)
    _report("layer-8k-local", compare(wl, g, r))
