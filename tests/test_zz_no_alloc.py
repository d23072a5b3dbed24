"""The allocation-free entry point, mkd_decode_step_static (the engine's workspace in the
library's static device array), against mkd_decode_step (a caller workspace) through the
C-ABI: two calls in a row, the second with a smaller batch, each compared with the
existing entry point on the same inputs (per-row relative error of the logits within
2e-2 and the same greedy tokens; the KV pools bit-identical, so the new slots agree
exactly) and with the CPU reference.  Needs an MI355X."""
import ctypes

import numpy as np
import pytest

import decode_megakernel_amd as mkd
import synth
from parity import REL_TOL, max_rel_rows, oracle_step

pytestmark = pytest.mark.gpu


def _run(eng, wl, static):
    import torch
    from synth import device as sdev

    pool = sdev.device_kv_pool(wl)
    inp = sdev.device_step_inputs(wl)
    logits = torch.full((wl.batch, wl.geom.vocab), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    eng.decode_step(inp["tokens"], inp["seq_lens"], inp["h_seq_lens"], inp["page_table"], pool, wl.n_pages,
                    logits, h_page_table=inp["h_page_table"], static=static)
    eng.sync_status()
    return logits.cpu().numpy(), sdev.bf16_bits(pool)


def test_static_entry_point_matches_workspace_entry_point():
    import torch
    from synth import device as sdev

    torch.cuda.set_device(0)
    calls = [synth.ragged_workload(synth.TINY, [33, 1, 100], spare_pages=3),
             synth.ragged_workload(synth.TINY, [15], spare_pages=3)]          # second call: smaller
    max_pages = max(wl.max_pages for wl in calls)
    W = sdev.device_weights(calls[0])
    ref_eng = mkd.Engine(synth.TINY, 0, max_batch=3, max_pages_per_seq=max_pages)
    ref_eng.load_weights(W)
    st_eng = mkd.Engine(synth.TINY, 0, max_batch=3, max_pages_per_seq=max_pages, workspace=False)
    st_eng.load_weights(W)
    assert 0 < st_eng.workspace_bytes() <= (64 << 20)
    for i, wl in enumerate(calls):
        print(f"[case] static entry point, call {i}, lengths {wl.seq_lens}", flush=True)
        a_logits, a_pool = _run(ref_eng, wl, static=False)
        b_logits, b_pool = _run(st_eng, wl, static=True)
        rel = max_rel_rows(b_logits, a_logits)
        print(f"[no-alloc] call {i}: logits rel {rel:.3g}, bit-equal {np.array_equal(a_logits, b_logits)}",
              flush=True)
        assert np.isfinite(b_logits).all() and rel <= REL_TOL
        assert np.array_equal(a_logits.argmax(-1), b_logits.argmax(-1))
        assert np.array_equal(a_pool, b_pool), "KV pools differ after the step"
        r = oracle_step(wl)
        assert max_rel_rows(b_logits, r["logits"]) <= REL_TOL
    ref_eng.close()
    st_eng.close()


def test_static_entry_point_rejects_oversized_workspace():
    # a geometry whose workspace exceeds the static array is refused before any launch
    eng = mkd.Engine(synth.FULL, 0, max_batch=16, max_pages_per_seq=24576, workspace=False)
    assert eng.workspace_bytes() > (64 << 20)
    fake = mkd.Weights(*([256] * 7))                 # recorded only: the call fails first
    assert mkd.lib().mkd_load_weights(eng._h, ctypes.byref(fake)) == mkd.MKD_OK
    one = np.zeros(1, np.int32)
    rc = mkd.lib().mkd_decode_step_static(eng._h, None, 1, 256, 256, one.ctypes.data, 256, None, 256, 1, 256)
    assert rc == mkd.MKD_ERR_CAPACITY
    assert b"MKD_STATIC_SCRATCH_BYTES" in mkd.lib().mkd_last_error(eng._h)
    eng.close()
