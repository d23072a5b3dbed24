"""Shared helpers of the GPU parity tests: run one decode step through the C-ABI and
the same step on the CPU reference from identical seeded inputs, and compare them
with the acceptance rules:

- hidden states and logits: per row, max|gpu - ref| / max|ref| <= 2e-2 (bf16
  weights, fp32 accumulation); the same bound per query-head row for the queries after
  RoPE and the attention output of every layer (each replayed by the reference layer
  function from the residual stream entering the layer), and per token for the
  routing weights;
- page-table / KV-slot indexing: bit-exact (every pool byte outside the written
  slots unchanged; written slots hold the bf16 of k and v);
- expert activations silu(gate) * up of the selected experts: the same bar per row;
- expert selection identical, except where the reference's gap between the k-th
  and (k+1)-th router logit is < 1e-3 (reported, not failed); the routing table the
  kernel publishes (active experts, per-expert token lists, entry records) bit-exact
  against the table derived from the selected ids;
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
    q: np.ndarray            # [L][B][nq*hd]
    attn: np.ndarray         # [L][B][nq*hd]
    route: np.ndarray        # [L][ROUTE_WORDS] int32
    act: np.ndarray          # [L][B*k][moe_inter]
    pool_after: np.ndarray   # uint16 bits
    pool_before: np.ndarray
    weights_bits: dict


def gpu_step(wl, mode=0, check_weights=False, schedule=None):
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
    if getattr(wl.geom, "attn_window", 0) > 0:
        eng.set_attention_window(wl.geom.attn_window, wl.geom.full_every)
    if schedule is not None:
        eng.set_schedule(*schedule)
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
        q=eng.debug_read(mkd.DEBUG_Q, wl.batch),
        attn=eng.debug_read(mkd.DEBUG_ATTN, wl.batch),
        route=eng.debug_read(mkd.DEBUG_ROUTE, wl.batch),
        act=eng.debug_read(mkd.DEBUG_ACT, wl.batch),
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


def route_table(ids, weights, k):
    """Expected routing-table words of one layer from the selected ids [B][k] and weights:
    choices and weights per token, active experts ascending, CSR offsets, entries
    (b*k + j) expert-major with tokens ascending, and each entry's (active index << 16 |
    position in its expert's list).  Layout of MKD_DEBUG_ROUTE in include/mkd.h."""
    ids = np.asarray(ids)
    B = ids.shape[0]
    t = np.zeros(1548, np.int64)
    for b in range(B):
        for j in range(k):
            t[b * 16 + j] = ids[b, j]
            t[256 + b * 16 + j] = int(np.asarray(weights[b, j], np.float32).view(np.int32))
    act = sorted(set(int(e) for e in ids.reshape(-1)))
    t[512] = len(act)
    at = 0
    for a, e in enumerate(act):
        t[520 + a] = e
        t[776 + a] = at
        pos = 0
        for b in range(B):
            for j in range(k):
                if ids[b, j] == e:
                    t[1036 + at] = b * k + j
                    t[1292 + b * k + j] = (a << 16) | pos
                    at += 1
                    pos += 1
    t[776 + len(act)] = at
    return t.astype(np.int64)


def check_route(table, ids, w, ref_ids, ref_w, ref_router, k):
    """One layer's routing against the reference: ids identical except near ties, weights
    within the bar where the ids agree, and the published table bit-exact (the lists
    derived from the kernel's own ids, which equal the reference's where no tie)."""
    rep = dict(topk_w_rel=0.0, ties=0)
    B = ids.shape[0]
    mism = np.any(ids != ref_ids, axis=-1)
    tie = router_near_tie(ref_router, k)
    assert not (mism & ~tie).any(), f"expert selection differs without a near tie: {np.argwhere(mism & ~tie)}"
    rep["ties"] = int((mism & tie).sum())
    same = ~mism
    if same.any():
        rep["topk_w_rel"] = max_rel_rows(w[same], ref_w[same])
        assert rep["topk_w_rel"] <= REL_TOL, rep
    exp = route_table(ids, w, k)
    got = np.asarray(table, np.int64) & 0xFFFFFFFF
    exp_u = exp & 0xFFFFFFFF
    n_ent = B * k
    words = np.r_[[512], 520 + np.arange(exp[512]), 776 + np.arange(exp[512] + 1), 1036 + np.arange(n_ent),
                  1292 + np.arange(n_ent)]
    assert np.array_equal(got[words], exp_u[words]), "published expert lists differ from the selected ids"
    choice = np.array([b * 16 + j for b in range(B) for j in range(k)])
    assert np.array_equal(got[choice], exp_u[choice]), "published choices differ from the selected ids"
    assert np.array_equal(got[256 + choice], exp_u[256 + choice]), "published weights differ from topk_w"
    if not mism.any():
        ref_tab = route_table(ref_ids, ref_w, k) & 0xFFFFFFFF
        assert np.array_equal(got[words], ref_tab[words]), "expert lists differ from the reference's"
    return rep


def check_attention(q, attn, ref_q, ref_attn, head_dim):
    """Queries after RoPE and attention outputs, per query-head row, within the bar."""
    rep = dict(q_rel=max_rel_rows(np.asarray(q).reshape(-1, head_dim), np.asarray(ref_q).reshape(-1, head_dim)),
               attn_rel=max_rel_rows(np.asarray(attn).reshape(-1, head_dim),
                                     np.asarray(ref_attn).reshape(-1, head_dim)))
    assert rep["q_rel"] <= REL_TOL and rep["attn_rel"] <= REL_TOL, rep
    return rep


def check_act(act, ids, x, w_gate_up, k):
    """Expert activations silu(gate) * up of every token's selected experts (the kernel's
    own choices, which equal the reference's except at near ties) against the reference
    expert activation on the reference's normalised input x [B][H]; per row within the bar.
    w_gate_up: one layer's [E][2I][H] bits."""
    ids = np.asarray(ids)
    B = ids.shape[0]
    worst = 0.0
    for b in range(B):
        for j in range(k):
            ref = oracle.expert_act(x[b], w_gate_up[ids[b, j]])
            worst = max(worst, max_rel_rows(act[b * k + j], ref))
    assert worst <= REL_TOL, dict(act_rel=worst)
    return dict(act_rel=worst)


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
    # per layer: queries, attention output and routing against the reference layer
    # function replayed from the reference residual stream (near ties of the reference's
    # router logits come from that replay)
    lay = reference_layers(wl, r)
    rep.update(q_rel=0.0, attn_rel=0.0, topk_w_rel=0.0, act_rel=0.0, router_ties=0)
    wgu = r["W"]["w_gate_up"].reshape(geo.n_layers, geo.n_experts, 2 * geo.moe_inter, geo.hidden)
    for layer in range(geo.n_layers):
        ac = check_act(g.act[layer], g.topk_ids[layer], lay["x"][layer], wgu[layer], geo.top_k)
        rep["act_rel"] = max(rep["act_rel"], ac["act_rel"])
        a = check_attention(g.q[layer], g.attn[layer], lay["q"][layer], lay["attn"][layer], geo.head_dim)
        rt = check_route(g.route[layer], g.topk_ids[layer], g.topk_w[layer], r["ids"][layer], r["w"][layer],
                         lay["router"][layer], geo.top_k)
        rep["q_rel"] = max(rep["q_rel"], a["q_rel"])
        rep["attn_rel"] = max(rep["attn_rel"], a["attn_rel"])
        rep["topk_w_rel"] = max(rep["topk_w_rel"], rt["topk_w_rel"])
        rep["router_ties"] += rt["ties"]
    # greedy argmax
    ga, ra = g.logits.argmax(-1), r["logits"].argmax(-1)
    srt = -np.sort(-r["logits"].astype(np.float64), axis=-1)
    band = REL_TOL * np.max(np.abs(r["logits"]), axis=-1)
    near = (srt[:, 0] - srt[:, 1]) < band
    rep["argmax_near_ties"] = int(((ga != ra) & near).sum())
    assert not ((ga != ra) & ~near).any(), "greedy argmax differs"
    return rep


def reference_layers(wl, r):
    """Reference intermediate values per layer (normalised input, queries, attention output,
    router logits),
    recomputed layer by layer with the reference layer function from the reference
    residual stream and the reference KV cache."""
    geo = wl.geom
    H = geo.hidden
    qd = geo.n_q_heads * geo.head_dim
    out = dict(x=np.empty((geo.n_layers, wl.batch, H), np.float32),
               q=np.empty((geo.n_layers, wl.batch, qd), np.float32),
               attn=np.empty((geo.n_layers, wl.batch, qd), np.float32),
               router=np.empty((geo.n_layers, wl.batch, geo.n_experts), np.float32))
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
                         W["w_down"].reshape(geo.n_layers, -1)[layer], h, debug=True, layer_index=layer)
        for key in out:
            out[key][layer] = o[key]
    assert np.array_equal(h, r["hidden"][geo.n_layers]), "layer replay differs from the reference step"
    return out
