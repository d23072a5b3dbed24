"""The continuous-decode loop on the GPU against the CPU reference: ragged sequences join
(their cached pages filled with fresh seeded K/V), are parked when the KV pool runs out of
pages and resume when pages return, and retire after their tokens.  Every step's logits
are replayed by the reference step from the batch the server reports (tokens fed, cache
positions, page-table rows) on a host mirror of the pool; greedy tokens agree except
near ties; at the end the pool matches the mirror (new slots within the bar, every other
byte exact).  Needs an MI355X."""
import numpy as np
import pytest

import decode_megakernel_amd as mkd
import oracle
import synth
from parity import REL_TOL, max_rel_rows

pytestmark = pytest.mark.gpu


def test_continuous_decode_join_park_retire():
    import torch
    from synth import device as sdev

    G = synth.TINY
    P, L, nkv, hd = G.page_size, G.n_layers, G.n_kv_heads, G.head_dim
    n_pages, max_batch, max_pages = 14, 4, 8
    wl = synth.make_workload("serve", G, [0], spare_pages=n_pages - 1, max_pages=max_pages)
    W = sdev.device_weights(wl)
    Wh = {k: sdev.bf16_bits(v) for k, v in W.items()}
    page_elems = nkv * P * hd
    host_pool = synth.host_normal_bf16(L * 2 * n_pages * page_elems, seed=77, stream=9, scale=1.0)
    pool = torch.from_numpy(host_pool.view(np.int16).copy()).cuda().view(torch.bfloat16)
    eng = mkd.Engine(G, 0, max_batch=max_batch, max_pages_per_seq=max_pages)
    eng.load_weights(W)
    srv = mkd.Server(eng, n_pages, max_live=6)
    rng = np.random.default_rng(5)
    pending = [(i, int(rng.integers(0, 60)), int(rng.integers(0, G.vocab)), int(rng.integers(1, 12)))
               for i in range(12)]
    want = {i: new for i, _, _, new in pending}
    written = {}     # page -> set of slots written by steps since the page was last filled
    last_tok = {}    # id -> token sampled at its last step
    generated = {i: 0 for i, *_ in pending}
    parked_seen, steps, ties, worst = 0, 0, 0, 0.0

    def fill(pages, salt):
        # fresh seeded K/V for a joining sequence's cached pages, on the mirror and the device
        for j, pg in enumerate(pages):
            vals = synth.host_normal_bf16(L * 2 * page_elems, seed=78 + salt, stream=9, scale=1.0,
                                          offset=j * L * 2 * page_elems)
            for blk in range(L * 2):
                a = (blk * n_pages + int(pg)) * page_elems
                host_pool[a:a + page_elems] = vals[blk * page_elems:(blk + 1) * page_elems]
                pool[a:a + page_elems] = torch.from_numpy(
                    vals[blk * page_elems:(blk + 1) * page_elems].view(np.int16).copy()).cuda().view(torch.bfloat16)
            written.pop(int(pg), None)

    while pending or srv.stats()["live"]:
        while pending:
            sid, clen, tok, new = pending[0]
            pages = srv.try_join(sid, clen, tok, new)
            if pages is None:
                break
            fill(pages, sid)
            pending.pop(0)
        torch.cuda.synchronize()
        print(f"[case] serve step {steps} {srv.stats()}", flush=True)
        n = srv.step(pool)
        parked_seen = max(parked_seen, srv.stats()["parked"])
        st = srv.last_step(logits=True)
        assert n == len(st["ids"]) > 0
        for b, sid in enumerate(st["ids"]):
            if int(sid) in last_tok:
                assert st["fed"][b] == last_tok[int(sid)], "a sequence was not fed its last sampled token"
            pos, row = int(st["seq_lens"][b]), st["page_table"][b]
            written.setdefault(int(row[pos // P]), set()).add(pos % P)
        ref, _, _, _ = oracle.decode_step(G, st["fed"], st["seq_lens"], st["page_table"], host_pool, n_pages, Wh,
                                          want_layers=False)
        worst = max(worst, max_rel_rows(st["logits"], ref))
        assert max_rel_rows(st["logits"], ref) <= REL_TOL
        ra = ref.argmax(-1)
        srt = -np.sort(-ref.astype(np.float64), axis=-1)
        near = (srt[:, 0] - srt[:, 1]) < REL_TOL * np.max(np.abs(ref), axis=-1)
        assert not ((st["sampled"] != ra) & ~near).any(), "greedy token differs"
        ties += int(((st["sampled"] != ra) & near).sum())
        assert (st["sampled"] == st["logits"].argmax(-1)).all(), "sampling kernel differs from argmax"
        for b, sid in enumerate(st["ids"]):
            last_tok[int(sid)] = int(st["sampled"][b])
            generated[int(sid)] += 1
        steps += 1
        assert steps < 200
    eng.sync_status()
    assert generated == want, "a sequence did not generate exactly its tokens"
    assert parked_seen > 0, "the pool never ran out: parking was not exercised"
    # the pool against the mirror: the slots steps wrote within the bar, the rest exact
    dev = sdev.bf16_bits(pool)
    mask = np.zeros(dev.size, bool)
    for pg, slots in written.items():
        for blk in range(L * 2):
            base = (blk * n_pages + pg) * page_elems
            for t in slots:
                if blk % 2 == 0:   # K: token-major [P][hd]
                    idx = base + np.arange(nkv)[:, None] * P * hd + t * hd + np.arange(hd)[None, :]
                else:              # V: dim-major [hd][P]
                    idx = base + np.arange(nkv)[:, None] * P * hd + np.arange(hd)[None, :] * P + t
                mask[idx.ravel()] = True
    assert np.array_equal(dev[~mask], host_pool[~mask]), "pool bytes outside the written slots differ"
    gk = oracle.bf16_to_f32(dev[mask]).astype(np.float64)
    rk = oracle.bf16_to_f32(host_pool[mask]).astype(np.float64)
    assert np.max(np.abs(gk - rk)) / max(np.max(np.abs(rk)), 1e-30) <= REL_TOL
    print(f"[serve] steps={steps} logits_rel={worst:.3g} near_ties={ties} max_parked={parked_seen}", flush=True)
    srv.close()
    eng.close()
