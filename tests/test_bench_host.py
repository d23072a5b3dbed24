"""Host logic of the benchmark: the algorithmic bytes a step must move (the roofline's
numerator), checked against hand counts.  No GPU."""
import dataclasses
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402
import synth  # noqa: E402


def _hand_count(g, seq_lens, distinct, windows):
    H, hd, nq, nkv, E, I, V = g.hidden, g.head_dim, g.n_q_heads, g.n_kv_heads, g.n_experts, g.moe_inter, g.vocab
    dense = ((nq + 2 * nkv) * hd * H + H * nq * hd + E * H + H) * 2
    expert = 3 * I * H * 2
    total = 0
    for layer in range(g.n_layers):
        w = windows[layer]
        kv = sum(min(s + 1, w) if w else s + 1 for s in seq_lens) * nkv * hd * 2 * 2
        total += dense + distinct[layer] * expert + kv
    return total + V * H * 2 + H * 2 + len(seq_lens) * H * 2


def test_algorithmic_bytes_full_attention():
    g = synth.FULL
    distinct = [8] * g.n_layers
    got = bench.algorithmic_bytes(g, [8192], distinct)
    assert got == _hand_count(g, [8192], distinct, [0] * g.n_layers)
    # 6.887 GB at exactly 8192 cached tokens (the benchmark's steps advance the position,
    # so its per-step average over the timed steps is slightly larger)
    assert abs(got / 1e9 - 6.8874) < 0.0001


def test_algorithmic_bytes_local_layers():
    # window 4096 on layers with (l + 1) % 4 != 0: those layers read at most 4096 positions
    g = dataclasses.replace(synth.FULL, attn_window=4096, full_every=4)
    lens = [8192, 100, 4095]
    distinct = list(range(8, 8 + g.n_layers))
    windows = [0 if (l + 1) % 4 == 0 else 4096 for l in range(g.n_layers)]
    assert bench.algorithmic_bytes(g, lens, distinct) == _hand_count(g, lens, distinct, windows)
    full = dataclasses.replace(g, attn_window=0)
    assert bench.algorithmic_bytes(g, lens, distinct) < bench.algorithmic_bytes(full, lens, distinct)
