"""The C-ABI library: loads without a GPU, exports every declared symbol, validates
its arguments, and builds schedules that pass the static checks.  CPU only."""
import ctypes
import os
import re

import numpy as np
import pytest

import decode_megakernel_amd as mkd
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OP_EMBED, OP_QKV, OP_ROUTER, OP_ATTN, OP_MOE_UP, OP_OUT, OP_LM_HEAD, OP_MOE_DOWN = range(1, 9)


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "mkd.h")).read()
    declared = set(re.findall(r"^\s*(?:int|void|size_t|const char\*)\s+(mkd_\w+)\s*\(", header, re.M))
    assert declared == set(mkd.EXPORTS)
    L = mkd.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_create_rejects_bad_geometry():
    bad = [dict(hidden=300), dict(head_dim=96), dict(page_size=8), dict(top_k=20),
           dict(n_q_heads=5)]
    for change in bad:
        g = synth.Geometry(**{**synth.TINY.__dict__, **change})
        with pytest.raises(mkd.MkdError) as ei:
            mkd.Engine(g, -1, 1, 8)
        assert ei.value.code == mkd.MKD_ERR_ARG
    with pytest.raises(mkd.MkdError):
        mkd.Engine(synth.TINY, -1, 17, 8)       # max_batch above 16


def test_host_engine_refuses_to_decode():
    e = mkd.Engine(synth.TINY, -1, 1, 8)
    rc = mkd.lib().mkd_decode_step(e._h, None, 1, None, None, None, None, None, None, 1, None)
    assert rc == mkd.MKD_ERR_STATE
    assert mkd.lib().mkd_sync_status(None) == mkd.MKD_ERR_ARG
    # a host-only engine has no workspace and refuses one
    assert mkd.lib().mkd_workspace_bytes(e._h) == 0
    assert mkd.lib().mkd_set_workspace(e._h, 256, 1 << 20) == mkd.MKD_ERR_STATE
    assert mkd.lib().mkd_set_watchdog(e._h, 0) == mkd.MKD_ERR_ARG
    assert mkd.lib().mkd_set_watchdog(e._h, 1000) == mkd.MKD_OK


def test_plan_rejects_oversized_output_tiles():
    # the output task holds (row, token) residual words two per lane: rt_rows * max_batch
    # <= 128 at the default 8 rows per tile holds for max_batch 16, the engine's limit
    with pytest.raises(mkd.MkdError):
        mkd.Engine(synth.FULL, -1, 17, 64)


def _waves(desc):
    return desc[:, 0], desc[:, 1]


GI = mkd.D_GIDX


@pytest.mark.parametrize("geom,max_batch,n_cu", [(synth.TINY, 1, 256), (synth.TINY, 3, 7),
                                                 (synth.FULL, 1, 256), (synth.FULL, 16, 256)])
def test_plan_structure(geom, max_batch, n_cu):
    e = mkd.Engine(geom, -1, max_batch, 64)
    desc, offs = e.plan(n_cu)
    assert len(offs) == n_cu + 1
    assert offs[0] == 0 and offs[-1] == desc.shape[0] and (np.diff(offs) >= 0).all()
    # every task in exactly one list, each list in global order; reserved words zero
    assert sorted(desc[:, GI].tolist()) == list(range(desc.shape[0]))
    assert (desc[:, GI + 1:] == 0).all()
    for li in range(n_cu):
        gidx = desc[offs[li]:offs[li + 1], GI]
        assert (np.diff(gidx) > 0).all()
    # round robin: CU c holds global indices c, c + n_cu, ...
    for cu in range(n_cu):
        assert (desc[offs[cu]:offs[cu + 1], GI] % n_cu == cu).all()
    ops = desc[:, 0]
    gq = geom.n_q_heads + 2 * geom.n_kv_heads
    n_rt = geom.hidden // 8
    assert (ops == OP_EMBED).sum() == n_rt
    assert (ops == OP_OUT).sum() == geom.n_layers * n_rt
    assert (ops == OP_LM_HEAD).sum() == -(-geom.vocab // 32)
    qkv = desc[ops == OP_QKV]
    # QKV tiles cover every (head, rope pair) exactly once per layer
    for layer in range(geom.n_layers):
        t = qkv[qkv[:, 1] == layer]
        covered = sorted((h, j0 + i) for h, j0, pb in t[:, 2:5] for i in range(pb))
        assert covered == [(h, i) for h in range(gq) for i in range(geom.head_dim // 2)]
    # queries and the K / V flags are tagged words: the attention claimers come after the
    # layer's QKV wave; ARG3 numbers the tiles of a head
    attn = desc[ops == OP_ATTN]
    for layer in range(geom.n_layers):
        a = attn[attn[:, 1] == layer]
        t = qkv[qkv[:, 1] == layer]
        assert a[:, GI].min() > t[:, GI].max()
        for h in range(gq):
            assert sorted(t[t[:, 2] == h][:, 5].tolist()) == list(range((t[:, 2] == h).sum()))
    # one MoE-down claimer per CU per layer after the layer's MoE-up claimers, when the
    # schedule's batches reach the split of the down rows out of the output tasks (2);
    # none for a batch-1 schedule
    if max_batch < 2:
        assert (ops == OP_MOE_DOWN).sum() == 0
    else:
        assert (ops == OP_MOE_DOWN).sum() == geom.n_layers * n_cu
        up, dn = desc[ops == OP_MOE_UP], desc[ops == OP_MOE_DOWN]
        for layer in range(geom.n_layers):
            assert dn[dn[:, 1] == layer][:, GI].min() > up[up[:, 1] == layer][:, GI].max()
    # one output task per residual row tile and layer; the residual rows travel as tagged
    # words and the next layer's tasks come after the output wave in the global order
    out = desc[ops == OP_OUT]
    for layer in range(geom.n_layers):
        o = out[out[:, 1] == layer]
        assert sorted(o[:, 2].tolist()) == list(range(n_rt))
        nxt = qkv[qkv[:, 1] == layer + 1] if layer + 1 < geom.n_layers else desc[ops == OP_LM_HEAD]
        assert nxt[:, GI].min() > o[:, GI].max()


def _task_key(d):
    # the descriptor without its wave and global indices (which the order renumbers)
    return tuple(int(v) for v in np.delete(d, [mkd.D_WAVE, GI]))


@pytest.mark.parametrize("geom", [synth.TINY, synth.FULL])
@pytest.mark.parametrize("order", [mkd.ORDER_DEFAULT, mkd.ORDER_ATTN_FIRST, mkd.ORDER_MOE_FIRST,
                                   mkd.ORDER_INTERLEAVED])
@pytest.mark.parametrize("placement", [mkd.PLACE_ROUND_ROBIN, mkd.PLACE_XCD])
def test_schedules_same_tasks_other_order(geom, order, placement):
    """Every named schedule deals the same tasks (same descriptors but for the global
    index) in the order and onto the workgroups it names, and passes the static checks."""
    n_cu = 256
    ref = mkd.Engine(geom, -1, 4, 64)
    d0, _ = ref.plan(n_cu)
    e = mkd.Engine(geom, -1, 4, 64)
    e.set_schedule(order, placement)
    desc, offs = e.plan(n_cu)
    assert sorted(_task_key(d) for d in desc) == sorted(_task_key(d) for d in d0)
    glob = desc[np.argsort(desc[:, GI])]
    ops, layers = glob[:, 0], glob[:, 1]
    for layer in range(geom.n_layers):
        pos = {op: np.nonzero((ops == op) & (layers == layer))[0]
               for op in (OP_QKV, OP_ROUTER, OP_ATTN, OP_MOE_UP, OP_MOE_DOWN, OP_OUT)}
        first = {op: p.min() for op, p in pos.items()}
        last = {op: p.max() for op, p in pos.items()}
        # producers ahead of consumers in every schedule
        assert last[OP_QKV] < first[OP_ATTN] and last[OP_ROUTER] < first[OP_MOE_UP]
        assert last[OP_MOE_UP] < first[OP_MOE_DOWN]
        assert max(last[OP_ATTN], last[OP_MOE_DOWN]) < first[OP_OUT]
        if order == mkd.ORDER_DEFAULT:
            assert last[OP_ROUTER] < first[OP_ATTN] and last[OP_ATTN] < first[OP_MOE_UP]
        elif order == mkd.ORDER_ATTN_FIRST:
            assert last[OP_ATTN] < first[OP_ROUTER]
        elif order == mkd.ORDER_MOE_FIRST:
            assert last[OP_ROUTER] < first[OP_QKV] and last[OP_MOE_DOWN] < first[OP_ATTN]
        else:
            # claimer i of the attention queue directly followed by claimer i of the MoE queue
            a, m = pos[OP_ATTN], pos[OP_MOE_UP]
            assert (glob[a, 2] == np.arange(len(a))).all() and (m - a == 1).all()
    for li in range(n_cu):
        g = desc[offs[li]:offs[li + 1], GI]
        assert (np.diff(g) > 0).all()
        q = g % n_cu
        if placement == mkd.PLACE_ROUND_ROBIN:
            assert (q == li).all()
        else:
            # XCD-major slots: workgroup li runs on XCD li mod 8 and takes the slots of its XCD
            assert ((q // (n_cu // 8)) == li % 8).all() and ((q % (n_cu // 8)) * 8 + q // (n_cu // 8) == li).all()


def test_schedule_rejects_bad_arguments():
    e = mkd.Engine(synth.TINY, -1, 1, 8)
    for order, placement in ((4, 0), (-1, 0), (0, 2)):
        assert mkd.lib().mkd_set_schedule(e._h, order, placement) == mkd.MKD_ERR_ARG
    e.set_schedule(mkd.ORDER_DEFAULT, mkd.PLACE_XCD)
    with pytest.raises(mkd.MkdError):
        e.plan(7)   # XCD placement needs a multiple of 8 compute units
    e.set_schedule(mkd.ORDER_DEFAULT, mkd.PLACE_ROUND_ROBIN)
    e.plan(7)


def test_attention_window_rejects_bad_arguments():
    e = mkd.Engine(synth.TINY, -1, 1, 8)
    for window, every in ((-1, 1), (4, 0), (4, -2)):
        with pytest.raises(RuntimeError):
            e.set_attention_window(window, every)
    e.set_attention_window(0, 1)
    e.set_attention_window(32, 4)
    e.close()
