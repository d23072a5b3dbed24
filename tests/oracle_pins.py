"""Pins of the CPU reference against facts fixed outside it: closed forms worked by
hand, invariants of the definitions, special cases that reduce to a library
routine (numpy / scipy / torch CPU), and brute force on tiny inputs.

Every check is a plain function that raises AssertionError on failure, so the
same list can be run against deliberately broken copies of the reference
(test_oracle_mutations.py) to show that each plausible mistake is caught.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os

import numpy as np
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# A tiny geometry with GQA group 2 and three KV groups of work (small and fast).
G = synth.Geometry(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, n_experts=6,
                   top_k=2, moe_inter=24, vocab=96, page_size=4)


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _rand_bf16(rng, shape, std=1.0):
    return _bf16(rng.standard_normal(shape).astype(np.float32) * std)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


# ------------------------------------------------------------------ bf16 conversion

def check_bf16_round_to_nearest_even():
    # Library pin: torch's float32 -> bfloat16 cast rounds to nearest even.
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 3,
                        np.array([1.0, 1.00390625, 1.01171875, -1.00390625, 0.0, 65504.0],
                                 np.float32)])
    got = np.array([oracle.lib().orc_f32_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, _bf16(x))
    # closed forms: the halfway cases round to the even neighbour
    assert oracle.lib().orc_f32_to_bf16(1.00390625) == 0x3F80
    assert oracle.lib().orc_f32_to_bf16(1.01171875) == 0x3F82
    assert oracle.bf16_to_f32(np.array([0x3F80, 0xC000], np.uint16)).tolist() == [1.0, -2.0]


# ------------------------------------------------------------------ matvec

def check_matvec_library():
    rng = np.random.default_rng(1)
    W = _rand_bf16(rng, (37, 150))
    x = rng.standard_normal(150).astype(np.float32)
    ref = oracle.bf16_to_f32(W).astype(np.float64) @ x.astype(np.float64)
    assert _rel(oracle.matvec(W, x), ref) < 1e-5


def check_matvec_one_hot_selects_column():
    rng = np.random.default_rng(2)
    W = _rand_bf16(rng, (9, 13))
    for c in (0, 7, 12):
        x = np.zeros(13, np.float32)
        x[c] = 1.0
        assert np.array_equal(oracle.matvec(W, x), oracle.bf16_to_f32(W[:, c]))


# ------------------------------------------------------------------ RMSNorm

def check_rmsnorm_closed_forms():
    ones = np.full(32, 0x3F80, np.uint16)
    # constant vector, eps 0: every entry becomes sign(c)
    out = oracle.rmsnorm(np.full(32, -3.5, np.float32), ones, 0.0)
    assert np.allclose(out, -1.0, atol=1e-6)
    # mean of squares of the output = ms / (ms + eps) with unit gamma
    rng = np.random.default_rng(3)
    v = rng.standard_normal(32).astype(np.float32)
    eps = 0.25
    ms = float(np.mean(v.astype(np.float64) ** 2))
    out = oracle.rmsnorm(v, ones, eps).astype(np.float64)
    assert abs(np.mean(out ** 2) - ms / (ms + eps)) < 1e-5


def check_rmsnorm_library_and_gamma():
    rng = np.random.default_rng(4)
    v = rng.standard_normal(64).astype(np.float32)
    gamma = _rand_bf16(rng, 64)
    eps = 1e-6
    ref = torch.nn.functional.rms_norm(torch.tensor(v, dtype=torch.float64), (64,),
                                       torch.tensor(oracle.bf16_to_f32(gamma), dtype=torch.float64),
                                       eps).numpy()
    assert _rel(oracle.rmsnorm(v, gamma, eps), ref) < 1e-5
    # scale invariance with eps = 0
    a = oracle.rmsnorm(v, gamma, 0.0)
    b = oracle.rmsnorm(v * 7.0, gamma, 0.0)
    assert _rel(a, b) < 1e-6


# ------------------------------------------------------------------ RoPE

def check_rope_worked_example():
    with open(os.path.join(GOLDEN, "rope_worked.json")) as f:
        fx = json.load(f)
    y = oracle.rope(np.array(fx["x"], np.float32), fx["base"], fx["pos"])
    assert np.allclose(y, fx["y"], atol=1e-6)


def check_rope_invariants():
    rng = np.random.default_rng(5)
    hd = 16
    q = rng.standard_normal(hd).astype(np.float32)
    k = rng.standard_normal(hd).astype(np.float32)
    assert np.array_equal(oracle.rope(q, 10000.0, 0), q)             # position 0: identity
    y = oracle.rope(q, 10000.0, 1234)
    half = hd // 2
    n0 = q[:half].astype(np.float64) ** 2 + q[half:].astype(np.float64) ** 2
    n1 = y[:half].astype(np.float64) ** 2 + y[half:].astype(np.float64) ** 2
    assert np.allclose(n0, n1, rtol=1e-5)                               # pair norms kept
    # the score depends only on the relative offset m - n
    d1 = float(np.dot(oracle.rope(q, 10000.0, 40), oracle.rope(k, 10000.0, 33)))
    d2 = float(np.dot(oracle.rope(q, 10000.0, 1007), oracle.rope(k, 10000.0, 1000)))
    assert abs(d1 - d2) < 1e-4 * max(1.0, abs(d1))


def check_rope_large_position():
    # At position 262144 pair 1 of a 4-dim head turns by 262144 * 10000^(-1/2)
    # = 2621.44 rad.  Angles formed in fp64 keep the rotation exact to fp32; an
    # fp32 product would be off by ~1e-4 rad.
    pos = 262144
    y = oracle.rope(np.array([0.0, 1.0, 0.0, 0.0], np.float32), 10000.0, pos)
    ang = pos * 10000.0 ** -0.5
    assert abs(float(y[1]) - math.cos(ang)) < 2e-7
    assert abs(float(y[3]) - math.sin(ang)) < 2e-7


# ------------------------------------------------------------------ paged attention

def _paged_pool(g, contiguous_k, contiguous_v, page_row, n_pages):
    """Scatter contiguous bf16 K/V [n_kv][n][hd] into a one-layer pool via the page
    table, using the layout stated in oracle.h (K token-major, V dim-major)."""
    P, D, nkv = g.page_size, g.head_dim, g.n_kv_heads
    pool = np.zeros(g.kv_layer_numel(n_pages), np.uint16)
    kview = pool[: n_pages * nkv * P * D].reshape(n_pages, nkv, P, D)
    vview = pool[n_pages * nkv * P * D:].reshape(n_pages, nkv, D, P)
    n = contiguous_k.shape[1]
    for t in range(n):
        page, tt = page_row[t // P], t % P
        for grp in range(nkv):
            kview[page, grp, tt, :] = contiguous_k[grp, t]
            vview[page, grp, :, tt] = contiguous_v[grp, t]
    return pool


def check_attention_worked_example():
    with open(os.path.join(GOLDEN, "attention_two_tokens.json")) as f:
        fx = json.load(f)
    g = dataclasses.replace(G, n_q_heads=1, n_kv_heads=1, head_dim=4, page_size=4)
    k = _bf16(np.array(fx["k"], np.float32))[None]
    v = _bf16(np.array(fx["v"], np.float32))[None]
    pool = _paged_pool(g, k, v, [2], 3)
    o = oracle.attention(g, 1, np.array([2], np.int32), pool, 3, np.array(fx["q"], np.float32))
    assert np.allclose(o, fx["o"], atol=1e-5)


def check_attention_paged_equals_contiguous():
    rng = np.random.default_rng(6)
    g = G
    n = 23                                                   # 6 pages, ragged last page
    n_pages = 11
    page_row = rng.permutation(n_pages)[:6].astype(np.int32)
    k = _rand_bf16(rng, (g.n_kv_heads, n, g.head_dim))
    v = _rand_bf16(rng, (g.n_kv_heads, n, g.head_dim))
    pool = _paged_pool(g, k, v, page_row, n_pages)
    q = rng.standard_normal(g.n_q_heads * g.head_dim).astype(np.float32)
    o = oracle.attention(g, n - 1, page_row, pool, n_pages, q)
    # library routine: scipy softmax over fp64 scores of the contiguous K/V
    grp = g.n_q_heads // g.n_kv_heads
    kf, vf = oracle.bf16_to_f32(k).astype(np.float64), oracle.bf16_to_f32(v).astype(np.float64)
    for j in range(g.n_q_heads):
        qj = q[j * g.head_dim:(j + 1) * g.head_dim].astype(np.float64)
        s = kf[j // grp] @ qj / math.sqrt(g.head_dim)
        ref = scipy.special.softmax(s) @ vf[j // grp]
        assert _rel(o[j * g.head_dim:(j + 1) * g.head_dim], ref) < 1e-5


def check_attention_special_cases():
    rng = np.random.default_rng(7)
    g = G
    n_pages = 5
    page_row = np.array([3, 1, 4, 0], np.int32)
    # one token: o = v of the head's own KV group, for every head (GQA mapping)
    k = _rand_bf16(rng, (g.n_kv_heads, 1, g.head_dim))
    v = _rand_bf16(rng, (g.n_kv_heads, 1, g.head_dim))
    pool = _paged_pool(g, k, v, page_row, n_pages)
    q = rng.standard_normal(g.n_q_heads * g.head_dim).astype(np.float32)
    o = oracle.attention(g, 0, page_row, pool, n_pages, q)
    grp = g.n_q_heads // g.n_kv_heads
    for j in range(g.n_q_heads):
        assert np.array_equal(o[j * g.head_dim:(j + 1) * g.head_dim],
                              oracle.bf16_to_f32(v[j // grp, 0]))
    # identical keys: o = mean of V
    n = 13
    k = np.repeat(_rand_bf16(rng, (g.n_kv_heads, 1, g.head_dim)), n, axis=1)
    v = _rand_bf16(rng, (g.n_kv_heads, n, g.head_dim))
    pool = _paged_pool(g, k, v, page_row, n_pages)
    o = oracle.attention(g, n - 1, page_row, pool, n_pages, q)
    for j in range(g.n_q_heads):
        ref = oracle.bf16_to_f32(v[j // grp]).astype(np.float64).mean(axis=0)
        assert _rel(o[j * g.head_dim:(j + 1) * g.head_dim], ref) < 1e-5


def check_attention_page_permutation_invariant():
    rng = np.random.default_rng(8)
    g = G
    n = 15
    n_pages = 9
    k = _rand_bf16(rng, (g.n_kv_heads, n, g.head_dim))
    v = _rand_bf16(rng, (g.n_kv_heads, n, g.head_dim))
    q = rng.standard_normal(g.n_q_heads * g.head_dim).astype(np.float32)
    outs = []
    for seed in range(3):
        row = np.random.default_rng(100 + seed).permutation(n_pages)[:4].astype(np.int32)
        pool = _paged_pool(g, k, v, row, n_pages)
        outs.append(oracle.attention(g, n - 1, row, pool, n_pages, q))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def check_attention_local_window_brute_force():
    # A local-attention layer attends to positions pos - W + 1 .. pos: scipy softmax over
    # exactly those positions of the contiguous K/V, for windows that start mid-page, on a
    # page boundary, cover one position, and exceed the sequence (every position).
    rng = np.random.default_rng(9)
    g = G
    n = 23
    n_pages = 11
    page_row = rng.permutation(n_pages)[:6].astype(np.int32)
    k = _rand_bf16(rng, (g.n_kv_heads, n, g.head_dim))
    v = _rand_bf16(rng, (g.n_kv_heads, n, g.head_dim))
    pool = _paged_pool(g, k, v, page_row, n_pages)
    q = rng.standard_normal(g.n_q_heads * g.head_dim).astype(np.float32)
    grp = g.n_q_heads // g.n_kv_heads
    kf, vf = oracle.bf16_to_f32(k).astype(np.float64), oracle.bf16_to_f32(v).astype(np.float64)
    pos = n - 1
    for window in (7, 8, 11, 1, 23, 40):
        o = oracle.attention(g, pos, page_row, pool, n_pages, q, window=window)
        t0 = max(0, pos - window + 1)
        for j in range(g.n_q_heads):
            qj = q[j * g.head_dim:(j + 1) * g.head_dim].astype(np.float64)
            s = kf[j // grp, t0:pos + 1] @ qj / math.sqrt(g.head_dim)
            ref = scipy.special.softmax(s) @ vf[j // grp, t0:pos + 1]
            assert _rel(o[j * g.head_dim:(j + 1) * g.head_dim], ref) < 1e-5, window
    # window 1: the new token's v exactly; window >= pos + 1: identical to full attention
    o1 = oracle.attention(g, pos, page_row, pool, n_pages, q, window=1)
    for j in range(g.n_q_heads):
        assert np.array_equal(o1[j * g.head_dim:(j + 1) * g.head_dim], oracle.bf16_to_f32(v[j // grp, pos]))
    assert np.array_equal(oracle.attention(g, pos, page_row, pool, n_pages, q, window=n),
                          oracle.attention(g, pos, page_row, pool, n_pages, q))


def check_local_layers_follow_full_every():
    # In a step, layer l is local iff (l + 1) % full_every != 0: a 2-layer geometry with
    # full_every 2 equals a step whose layer 0 runs with the window and layer 1 without
    # (each layer replayed with the layer function), and differs from the all-full step.
    rng = np.random.default_rng(10)
    base = dataclasses.replace(G, n_layers=2)
    loc = dataclasses.replace(base, attn_window=5, full_every=2)
    assert [oracle.layer_window(loc, l) for l in range(4)] == [5, 0, 5, 0]
    assert [oracle.layer_window(base, l) for l in range(2)] == [0, 0]
    wl = synth.ragged_workload(loc, [13, 6], spare_pages=1)
    W = synth.host_weights(wl)
    pt = synth.page_tables(wl)
    toks = synth.host_tokens(wl)
    pool = synth.host_kv_pool(wl)
    pool_full = pool.copy()
    logits, hl, _, _ = oracle.decode_step(loc, toks, wl.seq_lens, pt, pool, wl.n_pages, W)
    full, _, _, _ = oracle.decode_step(base, toks, wl.seq_lens, pt, pool_full, wl.n_pages, W)
    assert not np.allclose(logits, full)
    H = loc.hidden
    nl = loc.kv_layer_numel(wl.n_pages)
    rep = synth.host_kv_pool(wl)
    h = hl[0].copy()
    for layer in range(2):
        g_l = loc if layer == 0 else base
        oracle.layer(g_l, wl.seq_lens, pt, rep[layer * nl:(layer + 1) * nl], wl.n_pages, W["norm"][layer * H:(layer + 1) * H],
                     W["w_qkv"].reshape(2, -1)[layer], W["w_o"].reshape(2, -1)[layer], W["w_router"].reshape(2, -1)[layer],
                     W["w_gate_up"].reshape(2, -1)[layer], W["w_down"].reshape(2, -1)[layer], h,
                     layer_index=0 if layer == 0 else 1)
        assert np.array_equal(h, hl[layer + 1]), layer


# ------------------------------------------------------------------ routing

def check_topk_library_and_ties():
    rng = np.random.default_rng(9)
    for _ in range(20):
        r = np.round(rng.standard_normal(32) * 2, 1).astype(np.float32)   # many ties
        ids, w = oracle.topk_softmax(r, 5)
        ref = np.argsort(-r.astype(np.float64), kind="stable")[:5]       # ties: lower index
        assert np.array_equal(ids, ref)
        full = scipy.special.softmax(r.astype(np.float64))
        assert _rel(w, full[ref] / full[ref].sum()) < 1e-6
        assert abs(float(w.sum()) - 1.0) < 1e-6


# ------------------------------------------------------------------ experts

def check_expert_ffn_structured():
    # Diagonal gate/up and a permutation down-projection: y[perm[i]] ... closed form
    # y = P (silu(a * x) * (b * x)) with silu(z) = z * sigmoid(z) (scipy expit).
    rng = np.random.default_rng(10)
    H = I = 8
    a = rng.standard_normal(I).astype(np.float32)
    b = rng.standard_normal(I).astype(np.float32)
    a_bf, b_bf = _bf16(a), _bf16(b)
    gu = np.zeros((2 * I, H), np.uint16)
    gu[np.arange(I), np.arange(I)] = a_bf
    gu[I + np.arange(I), np.arange(I)] = b_bf
    perm = rng.permutation(I)
    dn = np.zeros((H, I), np.uint16)
    dn[perm, np.arange(I)] = 0x3F80           # y[perm[i]] = act[i]
    x = rng.standard_normal(H).astype(np.float64)
    af, bf = oracle.bf16_to_f32(a_bf).astype(np.float64), oracle.bf16_to_f32(b_bf).astype(np.float64)
    z = af * x
    act = z * scipy.special.expit(z) * (bf * x)
    ref = np.zeros(H)
    ref[perm] = act
    y = oracle.expert_ffn(x.astype(np.float32), gu, dn)
    assert _rel(y, ref) < 1e-5
    assert _rel(oracle.expert_act(x.astype(np.float32), gu), act) < 1e-5


def check_moe_equals_dense_masked_sum():
    rng = np.random.default_rng(11)
    g = G
    E, I, H = g.n_experts, g.moe_inter, g.hidden
    gu = _rand_bf16(rng, (E, 2 * I, H), 0.1)
    dn = _rand_bf16(rng, (E, H, I), 0.1)
    x = rng.standard_normal(H).astype(np.float32)
    ids = np.array([4, 1], np.int32)
    w = np.array([0.7, 0.3], np.float32)
    m = oracle.moe(g, x, ids, w, gu, dn)
    dense = np.zeros(H)
    for e in range(E):
        we = {4: 0.7, 1: 0.3}.get(e, 0.0)
        dense += np.float32(we) * oracle.expert_ffn(x, gu[e], dn[e]).astype(np.float64)
    assert _rel(m, dense) < 1e-6


# ------------------------------------------------------------------ layer / step

def _small_inputs(g, seq_lens, seed=12, n_spare=3):
    wl = synth.make_workload("pin", g, seq_lens, spare_pages=n_spare, weight_seed=seed,
                             kv_seed=seed + 1, token_seed=seed + 2)
    W = synth.host_weights(wl)
    pool = synth.host_kv_pool(wl)
    pt = synth.page_tables(wl)
    toks = synth.host_tokens(wl)
    return wl, W, pool, pt, toks


def check_kv_append_slot_and_untouched_bytes():
    g = G
    wl, W, pool, pt, toks = _small_inputs(g, [9, 4])
    before = pool.copy()
    logits, hl, ids, w = oracle.decode_step(g, toks, wl.seq_lens, pt, pool, wl.n_pages, W)
    changed = np.nonzero(pool != before)[0]
    allowed = set()
    nl = g.kv_layer_numel(wl.n_pages)
    for layer in range(g.n_layers):
        for b, pos in enumerate(wl.seq_lens):
            page, t = int(pt[b, pos // g.page_size]), pos % g.page_size
            for kv in (0, 1):
                for grp in range(g.n_kv_heads):
                    for e in range(g.head_dim):
                        allowed.add(layer * nl + oracle.kv_index(g, wl.n_pages, kv, page, grp, t, e))
    assert set(changed.tolist()) <= allowed
    # the written K of sequence 0, layer 0 is bf16(RoPE(W_k x)) with x the normed embedding
    H, hd, nq = g.hidden, g.head_dim, g.n_q_heads
    x = oracle.rmsnorm(oracle.bf16_to_f32(W["embed"].reshape(g.vocab, H)[toks[0]]),
                       W["norm"][:H], g.rms_eps)
    wq = W["w_qkv"].reshape(g.n_layers, g.qkv_rows, H)[0]
    kvec = oracle.bf16_to_f32(wq[nq * hd:(nq + 1) * hd]).astype(np.float64) @ x.astype(np.float64)
    kvec = oracle.rope(kvec.astype(np.float32), g.rope_base, wl.seq_lens[0])
    pos = wl.seq_lens[0]
    page, t = int(pt[0, pos // g.page_size]), pos % g.page_size
    got = np.array([pool[oracle.kv_index(g, wl.n_pages, 0, page, 0, t, e)] for e in range(hd)],
                   np.uint16)
    assert np.max(np.abs(oracle.bf16_to_f32(got) - kvec)) <= 1e-2 * np.max(np.abs(kvec))


def _rope_complex(y, base, pos):
    """Rotate-half RoPE written as complex multiplication: pair (i, i + hd/2) is the
    complex number y_i + j*y_{i+hd/2}, turned by the angle pos * base^(-2i/hd) (fp64)."""
    half = y.size // 2
    z = y[:half].astype(np.complex128) + 1j * y[half:].astype(np.float64)
    z *= np.exp(1j * pos * base ** (-2.0 * np.arange(half) / y.size))
    return np.concatenate([z.real, z.imag])


def check_qkv_rope_append_every_head():
    # Every output of the QKV step, against fp64 NumPy: q_j = RoPE(W_q[j] x, pos) for
    # every query head, and the slot written for every KV group holds bf16(RoPE(W_k[g] x,
    # pos)) in the K page and bf16(W_v[g] x) (no rotation) in the V page, read back
    # through the pool layout (K token-major, V dim-major).  Positions: the first slot of
    # a fresh page and a slot in the middle of a page.
    g = G
    rng = np.random.default_rng(14)
    H, hd, nq, nkv, P = g.hidden, g.head_dim, g.n_q_heads, g.n_kv_heads, g.page_size
    w = _rand_bf16(rng, (g.qkv_rows, H), 0.2)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    x = rng.standard_normal(H).astype(np.float32)
    y = wf @ x.astype(np.float64)
    n_pages = 7
    page_row = rng.permutation(n_pages)[:4].astype(np.int32)
    for pos in (8, 9):
        pool = _rand_bf16(rng, g.kv_layer_numel(n_pages))
        before = pool.copy()
        q = oracle.qkv_rope_append(g, pos, page_row, x, w, pool, n_pages)
        for j in range(nq):
            ref = _rope_complex(y[j * hd:(j + 1) * hd], g.rope_base, pos)
            assert _rel(q[j * hd:(j + 1) * hd], ref) < 1e-5, ("q head", j, pos)
        kview = pool[: n_pages * nkv * P * hd].reshape(n_pages, nkv, P, hd)
        vview = pool[n_pages * nkv * P * hd:].reshape(n_pages, nkv, hd, P)
        page, t = int(page_row[pos // P]), pos % P
        for grp in range(nkv):
            kref = _rope_complex(y[(nq + grp) * hd:(nq + grp + 1) * hd], g.rope_base, pos)
            vref = y[(nq + nkv + grp) * hd:(nq + nkv + grp + 1) * hd]
            kgot = oracle.bf16_to_f32(kview[page, grp, t, :]).astype(np.float64)
            vgot = oracle.bf16_to_f32(vview[page, grp, :, t]).astype(np.float64)
            # bf16 rounding: half an ulp, 2^-9 relative
            assert np.all(np.abs(kgot - kref) <= 2.0 ** -8 * np.abs(kref) + 1e-30), ("k group", grp, pos)
            assert np.all(np.abs(vgot - vref) <= 2.0 ** -8 * np.abs(vref) + 1e-30), ("v group", grp, pos)
        # nothing but the slot changed
        kview0 = before[: n_pages * nkv * P * hd].reshape(n_pages, nkv, P, hd)
        vview0 = before[n_pages * nkv * P * hd:].reshape(n_pages, nkv, hd, P)
        km = np.ones(kview.shape, bool)
        km[page, :, t, :] = False
        vm = np.ones(vview.shape, bool)
        vm[page, :, :, t] = False
        assert np.array_equal(kview[km], kview0[km]) and np.array_equal(vview[vm], vview0[vm])


def check_batch_equals_single_runs():
    g = G
    wl, W, pool, pt, toks = _small_inputs(g, [9, 4, 14])
    pool_b = pool.copy()
    logits, hl, _, _ = oracle.decode_step(g, toks, wl.seq_lens, pt, pool_b, wl.n_pages, W)
    for b in range(wl.batch):
        pool_1 = pool.copy()
        l1, h1, _, _ = oracle.decode_step(g, toks[b:b + 1], wl.seq_lens[b:b + 1], pt[b:b + 1],
                                          pool_1, wl.n_pages, W)
        assert np.array_equal(l1[0], logits[b])
        assert np.array_equal(h1[:, 0], hl[:, b])


def check_step_page_permutation_invariant():
    g = G
    wl, W, pool, pt, toks = _small_inputs(g, [10])
    l0, _, _, _ = oracle.decode_step(g, toks, wl.seq_lens, pt, pool.copy(), wl.n_pages, W)
    # relabel physical pages: pool' page sigma(p) holds pool page p
    sigma = np.random.default_rng(13).permutation(wl.n_pages)
    nl = g.kv_layer_numel(wl.n_pages)
    per_page = g.n_kv_heads * g.page_size * g.head_dim
    pool2 = np.empty_like(pool)
    src = pool.reshape(g.n_layers, 2, wl.n_pages, per_page)
    dst = pool2.reshape(g.n_layers, 2, wl.n_pages, per_page)
    dst[:, :, sigma, :] = src
    pt2 = np.where(pt >= 0, sigma[np.maximum(pt, 0)], -1).astype(np.int32)
    l1, _, _, _ = oracle.decode_step(g, toks, wl.seq_lens, pt2, pool2, wl.n_pages, W)
    assert np.array_equal(l0, l1)
    assert nl == pool.size // g.n_layers


def _random_gammas(g, seed):
    rng = np.random.default_rng(seed)
    return _bf16(1.0 + 0.5 * rng.standard_normal((g.n_layers + 1) * g.hidden))


def check_zero_branches_closed_form():
    # With W_o = 0 and W_down = 0 every layer leaves h unchanged, so the logits are
    # E . (rmsnorm(E[token]) * gamma_L) (numpy fp64 matmul).  Random gammas make
    # the final norm's gamma index matter.
    g = G
    wl, W, pool, pt, toks = _small_inputs(g, [6])
    W = dict(W)
    W["w_o"] = np.zeros_like(W["w_o"])
    W["w_down"] = np.zeros_like(W["w_down"])
    W["norm"] = _random_gammas(g, 21)
    logits, hl, _, _ = oracle.decode_step(g, toks, wl.seq_lens, pt, pool, wl.n_pages, W)
    E = oracle.bf16_to_f32(W["embed"]).reshape(g.vocab, g.hidden).astype(np.float64)
    gam = oracle.bf16_to_f32(W["norm"][g.n_layers * g.hidden:]).astype(np.float64)
    h = E[toks[0]]
    x = h / np.sqrt(np.mean(h ** 2) + g.rms_eps) * gam
    assert _rel(logits[0], E @ x) < 1e-5
    for layer in range(g.n_layers + 1):
        assert np.array_equal(hl[layer, 0], E[toks[0]].astype(np.float32))


def check_step_composition():
    # The step equals embedding -> layer 0 .. L-1 (each with its own weights, gamma_l
    # and KV slice) -> final norm with gamma_L -> tied LM head.
    g = G
    wl, W, pool, pt, toks = _small_inputs(g, [9, 3], seed=30)
    W = dict(W)
    W["norm"] = _random_gammas(g, 22)
    H = g.hidden
    pool_a = pool.copy()
    logits, hl, ids, w = oracle.decode_step(g, toks, wl.seq_lens, pt, pool_a, wl.n_pages, W)
    pool_b = pool.copy()
    nl = g.kv_layer_numel(wl.n_pages)
    h = oracle.bf16_to_f32(W["embed"].reshape(g.vocab, H)[toks]).copy()
    for layer in range(g.n_layers):
        assert np.array_equal(hl[layer], h)
        kvl = pool_b[layer * nl:(layer + 1) * nl]
        out = oracle.layer(g, wl.seq_lens, pt, kvl, wl.n_pages, W["norm"][layer * H:(layer + 1) * H],
                           W["w_qkv"].reshape(g.n_layers, -1)[layer],
                           W["w_o"].reshape(g.n_layers, -1)[layer],
                           W["w_router"].reshape(g.n_layers, -1)[layer],
                           W["w_gate_up"].reshape(g.n_layers, -1)[layer],
                           W["w_down"].reshape(g.n_layers, -1)[layer], h, debug=True)
        pool_b[layer * nl:(layer + 1) * nl] = kvl
        assert np.array_equal(ids[layer], out["ids"]) and np.array_equal(w[layer], out["w"])
    assert np.array_equal(hl[g.n_layers], h)
    assert np.array_equal(pool_a, pool_b)
    assert np.array_equal(logits, oracle.lm_head(g, h, W["norm"][g.n_layers * H:], W["embed"]))


def check_layer_composition():
    # One layer equals its composition from the step functions: rmsnorm, qkv+rope,
    # attention, O-proj, router, top-k, MoE, residual (each pinned above).
    g = G
    wl, W, pool, pt, toks = _small_inputs(g, [7])
    W = dict(W)
    W["norm"] = _random_gammas(g, 23)
    H = g.hidden
    h = oracle.bf16_to_f32(W["embed"].reshape(g.vocab, H)[toks]).copy()
    kv0 = pool[: g.kv_layer_numel(wl.n_pages)].copy()
    h_layer = h.copy()
    kv_a = kv0.copy()
    Wq = W["w_qkv"].reshape(g.n_layers, g.qkv_rows, H)[0]
    Wo = W["w_o"].reshape(g.n_layers, H, -1)[0]
    Wr = W["w_router"].reshape(g.n_layers, g.n_experts, H)[0]
    Wgu = W["w_gate_up"].reshape(g.n_layers, g.n_experts, 2 * g.moe_inter, H)[0]
    Wd = W["w_down"].reshape(g.n_layers, g.n_experts, H, g.moe_inter)[0]
    oracle.layer(g, wl.seq_lens, pt, kv_a, wl.n_pages, W["norm"][:H], Wq, Wo, Wr, Wgu, Wd, h_layer)
    kv_b = kv0.copy()
    x = oracle.rmsnorm(h[0], W["norm"][:H], g.rms_eps)
    q = oracle.qkv_rope_append(g, wl.seq_lens[0], pt[0], x, Wq, kv_b, wl.n_pages)
    o = oracle.attention(g, wl.seq_lens[0], pt[0], kv_b, wl.n_pages, q)
    a = oracle.matvec(Wo, o)
    ids, w = oracle.topk_softmax(oracle.matvec(Wr, x), g.top_k)
    m = oracle.moe(g, x, ids, w, Wgu, Wd)
    assert np.array_equal(kv_a, kv_b)
    assert np.array_equal(h_layer[0], h[0] + a + m)


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
