"""GPU parity: one decode step through the C-ABI against the CPU reference on the
same seeded inputs.  Needs an MI355X."""
import numpy as np
import pytest

import synth
from parity import compare, gpu_step, oracle_step

pytestmark = pytest.mark.gpu


def _report(name, rep):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                          for k, v in rep.items()), flush=True)


def test_tiny_step_megakernel():
    wl = synth.tiny_workload()
    print("[case] tiny b1 ctx64 megakernel", flush=True)
    g = gpu_step(wl, mode=0, check_weights=True)
    r = oracle_step(wl)
    for k, v in g.weights_bits.items():
        assert np.array_equal(v, r["W"][k]), f"GPU fill of {k} differs from the CPU fill"
    _report("tiny", compare(wl, g, r))


def test_tiny_step_op_per_kernel_matches_megakernel():
    wl = synth.tiny_workload()
    print("[case] tiny b1 ctx64 op-per-kernel", flush=True)
    a = gpu_step(wl, mode=1)
    b = gpu_step(wl, mode=0)
    r = oracle_step(wl)
    _report("tiny-ablation", compare(wl, a, r))
    assert np.array_equal(a.logits, b.logits)
    assert np.array_equal(a.hidden, b.hidden)


@pytest.mark.parametrize("seq_lens", [[0], [15], [16], [5, 64, 17, 0], [33, 1, 100],
                                      [5, 64, 17, 0, 33, 1, 100, 16], [3] * 16])
def test_tiny_ragged_batches(seq_lens):
    wl = synth.ragged_workload(synth.TINY, seq_lens, spare_pages=3)
    print(f"[case] tiny ragged {seq_lens}", flush=True)
    g = gpu_step(wl, mode=0)
    r = oracle_step(wl)
    _report(f"tiny-ragged-{seq_lens}", compare(wl, g, r))


def test_full_layer_8k():
    wl = synth.layer_workload(ctx=8192)
    print("[case] full-size layer b1 ctx8192", flush=True)
    g = gpu_step(wl, mode=0)
    r = oracle_step(wl)
    _report("layer-8k", compare(wl, g, r))
