"""Random-schedule model of how the recurrence kernel's loader and compute
waves meet through LDS flags (kda_recur.hip, tiles of four or more compute
waves), run on the CPU.

The rules modelled, with S = kSlots slots and LD loader waves:
  loader j owns chunks c = j, j + LD, ...; for c >= S it first waits until
  every compute wave's done word is >= c - S + 1 (all of them finished the
  slot's previous chunk, c - S); it then issues the chunk's loads into slot
  c mod S, waits for them to land, and sets ready[c mod S] = c + 1;
  compute wave w at step s waits until ready[s mod S] == s + 1, reads the slot
  (for a while), then sets done[w] = s + 1.
The model checks, under random interleavings and random load latencies, that
no slot is read before its chunk has landed, that no slot is overwritten while
a compute wave reads it, and that every wave finishes.  A deliberately lax
loader wait (one chunk too early) must be caught, which shows the check has
teeth."""
import random

import pytest


def simulate(WC, LD, S, steps, seed, lax=0):
    rnd = random.Random(seed)
    slot = [None] * S                 # (chunk, landed)
    ready = [0] * S
    done = [0] * WC
    loader = [{"c": j, "flight": False} for j in range(LD)]
    comp = [{"s": 0, "left": 0} for _ in range(WC)]   # left > 0: reading its slot
    for _ in range(2_000_000):
        actors = [("L", j) for j in range(LD) if loader[j]["c"] < steps]
        actors += [("C", w) for w in range(WC) if comp[w]["s"] < steps]
        if not actors:
            return
        kind, i = rnd.choice(actors)
        if kind == "L":
            st = loader[i]
            c = st["c"]
            if not st["flight"]:
                if c >= S and min(done) < c - S + 1 - lax:
                    continue
                for cs in comp:
                    if cs["left"] > 0 and cs["s"] % S == c % S:
                        raise AssertionError("slot %d overwritten while being read" % (c % S))
                slot[c % S] = (c, False)
                st["flight"] = True
            elif rnd.random() < 0.3:      # the chunk's loads land (vmcnt(0) returns)
                slot[c % S] = (c, True)
                ready[c % S] = c + 1
                st["c"], st["flight"] = c + LD, False
        else:
            cs = comp[i]
            s = cs["s"]
            if cs["left"] == 0:
                if ready[s % S] != s + 1:
                    continue
                if slot[s % S] != (s, True):
                    raise AssertionError("step %d read before its chunk landed" % s)
                cs["left"] = rnd.randint(1, 5)
            else:
                if slot[s % S] != (s, True):
                    raise AssertionError("slot of step %d changed while being read" % s)
                cs["left"] -= 1
                if cs["left"] == 0:
                    done[i] = s + 1
                    cs["s"] = s + 1
    raise AssertionError("no progress: the waves deadlocked")


# (compute waves, loaders, slots): the kernel's flag tiles (64 columns with a
# CU each: 4 / 4 / 6; 128 columns: 8 / 4 / 6) and other shapes of the rule
# kSlots = loaders + 2, plus tighter rings the rule must also survive.
SHAPES = [(4, 4, 6), (8, 4, 6), (4, 2, 4), (2, 6, 8), (4, 1, 3), (2, 2, 2), (4, 4, 4)]


@pytest.mark.parametrize("WC,LD,S", SHAPES)
def test_flag_protocol_is_safe_and_live(WC, LD, S):
    for steps in (0, 1, 2, 3, 5, 8, 17, 40):
        for seed in range(12):
            simulate(WC, LD, S, steps, seed)


def test_lax_loader_wait_is_caught():
    with pytest.raises(AssertionError, match="overwritten|changed|read before"):
        for seed in range(200):
            simulate(4, 4, 6, 40, seed, lax=1)
