"""Shared helpers of the GPU parity tests: run one decode step through the C-ABI and
the same step on the CPU reference from identical seeded inputs, and compare them
with the acceptance rules:

- hidden states and logits: per row, max|gpu - ref| / max|ref| <= 2e-2 (bf16
  weights, fp32 accumulation);
- page-table / KV-slot indexing: bit-exact (every pool byte outside the written
  slots unchanged; written slots hold the bf16 of k and v);
- expert selection identical, except where the reference's gap between the k-th
  and (k+1)-th router logit is < 1e-3 (reported, not failed);
- greedy argmax identical, except a near-tie of the reference's top two logits
  within the tolerance band (reported separately, never silently passed).
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import synth

REL_TOL = 2e-2
ROUTER_TIE = 1e-3


def max_rel_rows(gpu, ref):
    gpu = np.asarray(gpu, np.float64).reshape(-1, np.asarray(ref).shape[-1])
    ref = np.asarray(ref, np.float64).reshape(gpu.shape)
    num = np.max(np.abs(gpu - ref), axis=1)
    den = np.maximum(np.max(np.abs(ref), axis=1), 1e-30)
    return float(np.max(num / den))


@dataclasses.dataclass
class GpuStep:
    logits: np.ndarray
    hidden: np.ndarray       # [L+1][B][H]
    topk_ids: np.ndarray
    topk_w: np.ndarray
    router: np.ndarray
    pool_after: np.ndarray   # uint16 bits
    pool_before: np.ndarray
    weights_bits: dict


def gpu_step(wl, mode=0, check_weights=False):
    import torch

    import decode_megakernel_amd as mkd
    from synth import device as sdev

    W = sdev.device_weights(wl)
    pool = sdev.device_kv_pool(wl)
    inp = sdev.device_step_inputs(wl)
    torch.cuda.synchronize()
    pool_before = sdev.bf16_bits(pool)
    eng = mkd.Engine(wl.geom, 0, max_batch=wl.batch, max_pages_per_seq=wl.max_pages)
    eng.load_weights(W)
    eng.set_mode(mode)
    logits = torch.full((wl.batch, wl.geom.vocab), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    eng.decode_step(inp["tokens"], inp["seq_lens"], inp["h_seq_lens"], inp["page_table"], pool,
                    wl.n_pages, logits, h_page_table=inp["h_page_table"])
    eng.sync_status()
    out = GpuStep(
        logits=logits.cpu().numpy(),
        hidden=eng.debug_read(mkd.DEBUG_HIDDEN, wl.batch),
        topk_ids=eng.debug_read(mkd.DEBUG_TOPK_IDS, wl.batch),
        topk_w=eng.debug_read(mkd.DEBUG_TOPK_W, wl.batch),
        router=eng.debug_read(mkd.DEBUG_ROUTER, wl.batch),
        pool_after=sdev.bf16_bits(pool),
        pool_before=pool_before,
        weights_bits={k: sdev.bf16_bits(v) for k, v in W.items()} if check_weights else {},
    )
    eng.close()
    return out


def oracle_step(wl):
    W = synth.host_weights(wl)
    pool = synth.host_kv_pool(wl)
    pt = synth.page_tables(wl)
    toks = synth.host_tokens(wl)
    pool0 = pool.copy()
    logits, hl, ids, w = oracle.decode_step(wl.geom, toks, wl.seq_lens, pt, pool, wl.n_pages, W)
    return dict(W=W, pool_before=pool0, pool_after=pool, logits=logits, hidden=hl, ids=ids, w=w,
                page_table=pt, tokens=toks)


def written_slots(wl, pt):
    """Flat pool indices of the new token's k and v in every layer."""
    g = wl.geom
    nl = g.kv_layer_numel(wl.n_pages)
    P, D, nkv = g.page_size, g.head_dim, g.n_kv_heads
    idx = []
    for layer in range(g.n_layers):
        for b, pos in enumerate(wl.seq_lens):
            page, t = int(pt[b, pos // P]), pos % P
            for grp in range(nkv):
                kb = layer * nl + ((0 * wl.n_pages + page) * nkv + grp) * P * D
                vb = layer * nl + ((1 * wl.n_pages + page) * nkv + grp) * P * D
                idx.extend(kb + t * D + np.arange(D))
                idx.extend(vb + np.arange(D) * P + t)
    return np.asarray(idx, dtype=np.int64)


def router_near_tie(router_logits, k):
    """True where the gap between the k-th and (k+1)-th largest logit is < ROUTER_TIE."""
    s = -np.sort(-np.asarray(router_logits, np.float64), axis=-1)
    if s.shape[-1] <= k:
        return np.zeros(s.shape[:-1], bool)
    return (s[..., k - 1] - s[..., k]) < ROUTER_TIE


def compare(wl, g: GpuStep, r: dict):
    """Returns a dict of measured errors; raises AssertionError on a failed rule."""
    geo = wl.geom
    rep = {}
    rep["logits_rel"] = max_rel_rows(g.logits, r["logits"])
    rep["hidden_rel"] = max(max_rel_rows(g.hidden[l], r["hidden"][l]) for l in range(geo.n_layers + 1))
    assert np.isfinite(g.logits).all(), "non-finite logits"
    assert rep["hidden_rel"] <= REL_TOL, rep
    assert rep["logits_rel"] <= REL_TOL, rep
    # KV pool: bit-exact outside the written slots
    slots = written_slots(wl, r["page_table"])
    mask = np.ones(g.pool_after.size, bool)
    mask[slots] = False
    assert np.array_equal(g.pool_before, r["pool_before"]), "GPU and CPU pools differ before the step"
    assert np.array_equal(g.pool_after[mask], r["pool_before"][mask]), "bytes outside the new slots changed"
    gk = oracle.bf16_to_f32(g.pool_after[slots]).astype(np.float64)
    rk = oracle.bf16_to_f32(r["pool_after"][slots]).astype(np.float64)
    rep["kv_rel"] = float(np.max(np.abs(gk - rk)) / max(np.max(np.abs(rk)), 1e-30))
    assert rep["kv_rel"] <= REL_TOL, rep
    # routing
    mism = g.topk_ids != r["ids"]
    tie = np.zeros(mism.shape[:2], bool)
    # recompute the reference router logits' near ties from the GPU logits' order is not
    # allowed; the reference layer function gives them exactly
    rep["topk_mismatch_rows"] = int(np.any(mism, axis=-1).sum())
    rep["router_ties"] = 0
    if rep["topk_mismatch_rows"]:
        ref_router = reference_router_logits(wl, r, g)
        tie = router_near_tie(ref_router, geo.top_k)
        bad = np.any(mism, axis=-1) & ~tie
        rep["router_ties"] = int((np.any(mism, axis=-1) & tie).sum())
        assert not bad.any(), f"expert selection differs without a near-tie: {np.argwhere(bad)}"
    # greedy argmax
    ga, ra = g.logits.argmax(-1), r["logits"].argmax(-1)
    srt = -np.sort(-r["logits"].astype(np.float64), axis=-1)
    band = REL_TOL * np.max(np.abs(r["logits"]), axis=-1)
    near = (srt[:, 0] - srt[:, 1]) < band
    rep["argmax_near_ties"] = int(((ga != ra) & near).sum())
    assert not ((ga != ra) & ~near).any(), "greedy argmax differs"
    return rep


def reference_router_logits(wl, r, g):
    """Reference router logits per layer, recomputed layer by layer with the reference
    layer function from the reference residual stream."""
    geo = wl.geom
    H = geo.hidden
    out = np.empty((geo.n_layers, wl.batch, geo.n_experts), np.float32)
    pool = r["pool_before"].copy()
    nl = geo.kv_layer_numel(wl.n_pages)
    W = r["W"]
    h = r["hidden"][0].copy()
    for layer in range(geo.n_layers):
        kvl = pool[layer * nl:(layer + 1) * nl]
        o = oracle.layer(geo, wl.seq_lens, r["page_table"], kvl, wl.n_pages, W["norm"][layer * H:(layer + 1) * H],
                         W["w_qkv"].reshape(geo.n_layers, -1)[layer], W["w_o"].reshape(geo.n_layers, -1)[layer],
                         W["w_router"].reshape(geo.n_layers, -1)[layer],
                         W["w_gate_up"].reshape(geo.n_layers, -1)[layer],
                         W["w_down"].reshape(geo.n_layers, -1)[layer], h, debug=True)
        out[layer] = o["router"]
    return out
