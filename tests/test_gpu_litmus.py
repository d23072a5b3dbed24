"""Litmus test of the inter-workgroup protocol across XCDs (mkd_protocol_litmus): 128
producer / consumer pairs of workgroups on different XCDs, 2000 rounds over the same
buffers with the step's own primitives.  No tagged word may carry a new tag with an old
value, no data published before a flag may be read stale after the flag and an acquire,
and every wait must complete.  Needs an MI355X."""
import pytest

import decode_megakernel_amd as mkd

pytestmark = pytest.mark.gpu


def test_message_passing_across_xcds():
    n_pairs, rounds = 128, 2000
    print(f"[case] litmus {n_pairs} pairs x {rounds} rounds", flush=True)
    r = mkd.protocol_litmus(0, n_pairs, rounds)
    print(f"[litmus] {r}", flush=True)
    assert r["timeouts"] == 0 and r["rounds_done"] == n_pairs * rounds
    assert r["torn_words"] == 0, "a tagged word carried a new tag with an old value"
    assert r["stale_data"] == 0, "data published before a flag was read stale after the flag and an acquire"
