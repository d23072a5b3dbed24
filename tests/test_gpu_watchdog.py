"""The kernel's bounded waits (section "Barriers": every waiter spins until its dependency
is met; here each wait is bounded by the engine's watchdog).  With a watchdog of one poll,
forced from the host, the step's first wait on data that has not arrived gives up: the
step reports MKD_ERR_DEADLOCK and every workgroup leaves (the kernel ends).  The engine is
then usable again: with the default watchdog the same step on the same pool gives output
identical to a fresh engine's, which matches the CPU reference.  Needs an MI355X."""
import numpy as np
import pytest

import decode_megakernel_amd as mkd
import synth
from parity import REL_TOL, gpu_step, max_rel_rows, oracle_step

pytestmark = pytest.mark.gpu


def test_watchdog_gives_up_and_engine_recovers():
    import torch
    from synth import device as sdev

    wl = synth.tiny_workload()
    W = sdev.device_weights(wl)
    pool = sdev.device_kv_pool(wl)
    inp = sdev.device_step_inputs(wl)
    eng = mkd.Engine(wl.geom, 0, max_batch=wl.batch, max_pages_per_seq=wl.max_pages)
    eng.load_weights(W)
    logits = torch.full((wl.batch, wl.geom.vocab), float("nan"), dtype=torch.float32, device="cuda")

    def step():
        eng.decode_step(inp["tokens"], inp["seq_lens"], inp["h_seq_lens"], inp["page_table"], pool,
                        wl.n_pages, logits, h_page_table=inp["h_page_table"])
        torch.cuda.synchronize()
        return mkd.lib().mkd_sync_status(eng._h)

    eng.set_watchdog(1)
    codes = []
    for i in range(3):
        print(f"[case] watchdog 1 poll, step {i}", flush=True)
        codes.append(step())
    print(f"[watchdog] status codes with one poll: {codes}", flush=True)
    assert set(codes) <= {mkd.MKD_OK, mkd.MKD_ERR_DEADLOCK}
    assert mkd.MKD_ERR_DEADLOCK in codes, "no wait gave up with a one-poll watchdog"
    eng.set_watchdog(4000000)
    print("[case] default watchdog after the failed steps", flush=True)
    assert step() == mkd.MKD_OK
    got_logits = logits.cpu().numpy()
    got_hidden = eng.debug_read(mkd.DEBUG_HIDDEN, wl.batch)
    eng.close()
    fresh = gpu_step(wl)
    assert np.array_equal(got_logits, fresh.logits) and np.array_equal(got_hidden, fresh.hidden)
    r = oracle_step(wl)
    assert max_rel_rows(got_logits, r["logits"]) <= REL_TOL
