"""Seeded synthetic inputs: generator statistics, determinism, page-table validity.
CPU only (the GPU fill is compared with the CPU fill in the GPU tests)."""
import numpy as np
import torch

import synth


def test_normal_statistics_and_determinism():
    a = synth.host_normal_f32(200000, seed=5, stream=3, scale=1.0)
    assert abs(float(a.mean())) < 0.01 and abs(float(a.std()) - 1.0) < 0.01
    assert np.array_equal(a, synth.host_normal_f32(200000, seed=5, stream=3, scale=1.0))
    # counter-based: an offset window equals the corresponding slice
    b = synth.host_normal_f32(1000, seed=5, stream=3, scale=1.0, offset=12345)
    assert np.array_equal(b, a[12345:13345])
    assert not np.array_equal(a[:1000], synth.host_normal_f32(1000, seed=6, stream=3, scale=1.0))


def test_bf16_fill_is_rounded_f32_fill():
    f = synth.host_normal_f32(50000, seed=1, stream=4, scale=0.02)
    h = synth.host_normal_bf16(50000, seed=1, stream=4, scale=0.02)
    ref = torch.tensor(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, ref)
    assert abs(float(f.std()) - 0.02) < 0.001


def test_page_tables_valid():
    for wl in (synth.tiny_workload(), synth.layer_workload(),
               synth.ragged_workload(synth.TINY, [5, 64, 17, 0], spare_pages=4)):
        pt = synth.page_tables(wl)
        assert pt.shape == (wl.batch, wl.max_pages)
        used = []
        for b, s in enumerate(wl.seq_lens):
            n = (s + 1 + wl.geom.page_size - 1) // wl.geom.page_size
            row = pt[b, :n]
            assert (row >= 0).all() and (row < wl.n_pages).all()
            used.extend(row.tolist())
        assert len(used) == len(set(used))          # no page shared between sequences


def test_tokens_in_vocab():
    wl = synth.ragged_workload(synth.TINY, [3] * 16)
    t = synth.host_tokens(wl)
    assert t.dtype == np.int32 and ((t >= 0) & (t < wl.geom.vocab)).all()


def test_gains_differ_from_one_and_per_layer():
    g = synth.host_gains(100000, seed=0)
    f = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(f.mean() - 1.0) < 0.01 and abs(f.std() - 0.25) < 0.01
    assert (g != 0x3F80).mean() > 0.95
    # counter-based, like the other streams
    assert np.array_equal(synth.host_gains(500, seed=0, offset=2048), g[2048:2548])
    # equal to bf16(1 + 0.25 * deviate) of the f32 normal stream
    n = synth.host_normal_f32(1000, seed=0, stream=synth.STREAM["norm"], scale=0.25)
    ref = torch.tensor(1.0 + n.astype(np.float64)).to(torch.float32).to(torch.bfloat16)
    assert np.array_equal(g[:1000], ref.view(torch.int16).numpy().view(np.uint16))
