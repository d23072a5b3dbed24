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

OP_EMBED, OP_QKV, OP_ROUTER, OP_ATTN, OP_MOE_UP, OP_OUT, OP_LM_HEAD = range(1, 8)


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
    # one output task per residual row tile and layer; the residual rows travel as tagged
    # words and the next layer's tasks come after the output wave in the global order
    out = desc[ops == OP_OUT]
    for layer in range(geom.n_layers):
        o = out[out[:, 1] == layer]
        assert sorted(o[:, 2].tolist()) == list(range(n_rt))
        nxt = qkv[qkv[:, 1] == layer + 1] if layer + 1 < geom.n_layers else desc[ops == OP_LM_HEAD]
        assert nxt[:, GI].min() > o[:, GI].max()
