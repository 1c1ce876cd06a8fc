"""Host model of the half-stage ring of the 8-wave core (Tile8H in
test_weight_mlp_amd/csrc/mfma_core.h), checked for every K loop length the
library can run: each half stage is loaded exactly once, into a slot that no
wave still reads and that holds no half still in flight, and the vector-memory
wait at the top of every stage (the counter retires a wave's loads in issue
order) covers both halves of that stage.

The model follows the kernel's schedule: halves B0 A0 B1 A1 ... (half h is
stage h // 2, B when h is even) in slot h % 5; halves 0-2 issued before the
loop; stage s waits until at most NBL loads are pending (none at the last
stage), passes the LDS barrier, and issues half 2s+3 (k-steps 0-1), then half
2s+4 (k-steps 2-3), halves of stages past the end being skipped.
"""
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NSLOT = 5


def _core_source():
    with open(os.path.join(ROOT, "test_weight_mlp_amd", "csrc", "mfma_core.h")) as fh:
        return fh.read()


def test_model_matches_the_kernel_schedule():
    # the schedule constants the model assumes, as the kernel writes them
    src = _core_source()
    body = src[src.index("struct Tile8H"):]
    for anchor in ("NSLOT = 5", "for (int h = 0; h < 3; ++h) issue_half(", "if (s + 1 < S) wait_vmcnt<NBL>();",
                   "issue_half(oa, ob, lds, 2 * s + 3, S,", "issue_half(oa, ob, lds, 2 * s + 4, S,",
                   "((2 * s + 1) % NSLOT) * SLOT", "((2 * s) % NSLOT) * SLOT"):
        assert anchor in body, anchor


def _run(S, na, nbl):
    issued = []          # one entry per load instruction of this wave: its half
    slot_of = {}         # slot -> half it holds (issued, not yet dead)
    read_done = set()    # halves whose stage has been multiplied

    def issue(h):
        if h // 2 >= S:
            return
        slot = h % NSLOT
        prev = slot_of.get(slot)
        # the slot's previous half must have been read by every wave already
        assert prev is None or prev in read_done, (S, h, prev)
        assert h not in issued, (S, h)
        slot_of[slot] = h
        issued.extend([h] * (nbl if h % 2 == 0 else na))

    for h in range(3):
        issue(h)
    for s in range(S):
        pending = nbl if s + 1 < S else 0
        done = issued[:len(issued) - pending] if pending else list(issued)
        for h in (2 * s, 2 * s + 1):
            # every load instruction of the half has retired
            assert issued.count(h) > 0 and done.count(h) == issued.count(h), (S, s, h)
        # the barrier: stage s-1 has been read by every wave
        if s > 0:
            read_done.update((2 * s - 2, 2 * s - 1))
        reading = {(2 * s) % NSLOT, (2 * s + 1) % NSLOT}
        in_flight = {(2 * s + 2) % NSLOT} if s + 1 < S else set()
        for h in (2 * s + 3, 2 * s + 4):
            if h // 2 < S:
                assert h % NSLOT not in reading | in_flight, (S, s, h)
            issue(h)
    # every half of every stage went out exactly once
    assert sorted(set(issued)) == list(range(2 * S))


@pytest.mark.parametrize("S", list(range(1, 41)) + [152, 153])
def test_ring_schedule(S):
    # 256 x 256 tiles: 4 load instructions a wave for either part
    _run(S, na=4, nbl=4)
    # the wait counts hold for unequal parts too
    _run(S, na=2, nbl=6)
