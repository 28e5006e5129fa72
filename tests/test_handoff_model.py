"""A CPU model of the draw kernel's hand-off between the splits of a chain (no GPU).

Protocol, per split s of a chain with S splits:
  1. store its candidate (two 64-bit words) with write-through agent-scope stores;
  2. wait until its own stores are acknowledged (s_waitcnt vmcnt(0));
  3. increment the chain's counter (agent-scope atomic, returns the old value);
  4. the split that read S - 1 reads every split's candidate with coherent loads
     and picks the token.

The model lets every store sit unacknowledged (invisible to other splits) for an
arbitrary time until its owner's wait, and interleaves the splits' steps at
random; the atomic itself is indivisible, as on the hardware. It checks that
exactly one split selects and that it always sees every candidate, and that the
same search finds a stale read once the wait is taken out (a planted mistake),
so the wait is what the protocol rests on.
"""
import random

import pytest


def run(S: int, rng: random.Random, with_wait: bool) -> tuple[int, bool]:
    """One interleaving. Returns (number of selecting splits, selector saw all)."""
    memory = {}                      # visible words: (split, word) -> value
    pending = {s: [] for s in range(S)}  # stores issued but not yet acknowledged
    counter = [0]
    step = {s: 0 for s in range(S)}
    selectors, saw_all = 0, True
    live = list(range(S))
    while live:
        s = rng.choice(live)
        # any unacknowledged store may become visible at any moment
        for o in range(S):
            if pending[o] and rng.random() < 0.3:
                key, val = pending[o].pop(0)
                memory[key] = val
        st = step[s]
        if st == 0:                  # two stores, both pending until acknowledged
            pending[s] += [((s, 0), 1000 + s), ((s, 1), s)]
            step[s] = 1 if with_wait else 2
        elif st == 1:                # wait: the stores complete before going on
            for key, val in pending[s]:
                memory[key] = val
            pending[s].clear()
            step[s] = 2
        elif st == 2:                # the counter's atomic increment
            prev = counter[0]
            counter[0] += 1
            step[s] = 3 if prev == S - 1 else 4
        elif st == 3:                # the last arriver reads every candidate
            selectors += 1
            seen = [(memory.get((o, 0)), memory.get((o, 1))) for o in range(S)]
            saw_all = saw_all and all(v == (1000 + o, o) for o, v in enumerate(seen))
            step[s] = 4
        if step[s] == 4:
            live.remove(s)
    return selectors, saw_all


@pytest.mark.parametrize("S", [2, 3, 16])
def test_last_arriver_sees_every_candidate(S):
    rng = random.Random(100 + S)
    for _ in range(3000):
        selectors, saw_all = run(S, rng, with_wait=True)
        assert selectors == 1
        assert saw_all


def test_without_the_wait_a_stale_read_is_found():
    rng = random.Random(7)
    stale = 0
    for _ in range(3000):
        selectors, saw_all = run(4, rng, with_wait=False)
        assert selectors == 1
        stale += not saw_all
    assert stale > 0
