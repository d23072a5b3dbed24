"""The continuous-decode loop's scheduling, checked without a GPU (a server over a
host-only engine does every step's bookkeeping without launching): join order, batch
limit, page allocation on page boundaries, parking when the pool is exhausted and
resuming when pages return, retirement, and the capacity and argument errors."""
import numpy as np
import pytest

import decode_megakernel_amd as mkd
import synth

P = synth.TINY.page_size


def _server(n_pages, max_batch=2, max_live=8, max_pages=8):
    e = mkd.Engine(synth.TINY, -1, max_batch, max_pages)
    return e, mkd.Server(e, n_pages, max_live)


def test_join_allocates_cached_pages_lowest_first():
    e, s = _server(10)
    assert list(s.join(1, 2 * P + 3, 5, 4)) == [0, 1, 2]
    assert list(s.join(2, 0, 6, 1)) == []
    assert s.stats() == dict(live=2, parked=0, free_pages=7)


def test_steps_feed_positions_and_retire():
    e, s = _server(10, max_batch=2)
    s.join(10, P - 1, 7, 2)    # next token at the last slot of page 0, then opens page 1
    s.join(11, 0, 8, 1)        # empty cache: its first token opens page 0
    assert s.step(None) == 2
    st = s.last_step()
    assert list(st["ids"]) == [10, 11] and list(st["seq_lens"]) == [P - 1, 0]
    assert list(st["fed"]) == [7, 8]           # first tokens; later tokens come from sampling
    assert list(st["page_table"][0][:1]) == [0] and st["page_table"][0][1] == -1
    assert st["page_table"][1][0] == 1         # the new sequence's page for position 0
    # sequence 11 generated its one token and retired; its page is free again
    assert s.stats() == dict(live=1, parked=0, free_pages=9)
    assert s.step(None) == 1
    st = s.last_step()
    assert list(st["seq_lens"]) == [P] and list(st["fed"]) == [-1]
    assert list(st["page_table"][0][:2]) == [0, 1]   # page 1 (returned by 11) opened for position P
    assert s.stats() == dict(live=0, parked=0, free_pages=10)
    assert s.step(None) == 0


def test_batch_limit_keeps_join_order():
    e, s = _server(20, max_batch=2)
    for i in range(4):
        s.join(i, 3, 1, 1)
    assert s.step(None) == 2 and list(s.last_step()["ids"]) == [0, 1]
    assert s.step(None) == 2 and list(s.last_step()["ids"]) == [2, 3]
    assert s.stats()["live"] == 0


def test_park_and_resume():
    e, s = _server(3, max_batch=2)
    s.join(1, P, 1, 3)        # holds page 0; its first token opens a page
    s.join(2, P, 1, 3)        # holds page 1
    assert s.step(None) == 1  # 1 takes page 2, 2 finds no free page and is parked
    assert list(s.last_step()["ids"]) == [1]
    assert s.stats() == dict(live=2, parked=1, free_pages=0)
    assert s.step(None) == 1 and s.step(None) == 1   # 1 finishes; pages 0 and 2 return
    assert s.stats() == dict(live=1, parked=1, free_pages=2)
    assert s.step(None) == 1                         # 2 resumes on a returned page
    st = s.last_step()
    assert list(st["ids"]) == [2] and list(st["seq_lens"]) == [P] and st["page_table"][0][1] in (0, 2)
    assert s.stats()["parked"] == 0


def test_all_parked_is_a_capacity_error():
    e, s = _server(2, max_batch=2)
    s.join(1, P, 1, 2)
    s.join(2, P, 1, 2)
    with pytest.raises(mkd.MkdError) as ei:
        s.step(None)
    assert ei.value.code == mkd.MKD_ERR_CAPACITY
    assert s.stats() == dict(live=2, parked=2, free_pages=0)


def test_join_errors():
    e, s = _server(4, max_live=2, max_pages=8)
    assert s.try_join(1, 5 * P, 1, 1) is None          # more pages than free: nothing taken
    assert s.stats()["free_pages"] == 4
    with pytest.raises(mkd.MkdError):
        s.join(1, 8 * P, 1, 1)                          # longer than max_pages_per_seq pages
    with pytest.raises(mkd.MkdError):
        s.join(1, 0, synth.TINY.vocab, 1)               # token id out of range
    s.join(1, 0, 1, 1)
    with pytest.raises(mkd.MkdError):
        s.join(1, 0, 1, 1)                              # duplicate id
    s.join(2, 0, 1, 1)
    assert s.try_join(3, 0, 1, 1) is None               # max_live
