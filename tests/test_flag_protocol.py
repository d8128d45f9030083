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


# ---------------------------------------------------------------------------
# The fused kernel (kda_fused.hip): four prep waves build the chunk records in
# phases, four recurrence waves consume them, all meeting through flags.
#
# Steps s = -5 .. nch - 1; a flag holds s + 6 once its wave finished step s.
# Shared buffers and their contents:
#   group slot (g + 5) mod D: group g = raw inputs of chunk g + 5 (read by prep
#     wave (g + 5) mod 4 in phase 0 at step g) and value rows of chunk g (read
#     by the recurrence waves at step g); loaded by that prep wave, issued at
#     step g - D + 1, landed by the top of step g;
#   record slot c mod 6: chunk c, written by prep wave c mod 4 in phases 0..3
#     at steps c - 5 .. c - 2, its T written by the recurrence waves at step
#     c - 1 (one part each), read whole by the recurrence waves at step c;
#   lts[c mod 2]: L of chunk c, written in phase 3 (step c - 2), read by the
#     recurrence waves' inverse at step c - 1.
# Rules (the kernel's waits):
#   prep p, step s: if it loaded group s, wait for it and set gready; wait
#     until every recurrence wave finished step s - 1; before issuing group
#     s + D - 1 (if its own), wait until prep wave (s + 4) mod 4 finished step
#     s - 1; do the phase; set pdone.
#   recurrence w, step -1: wait pdone[0] >= 4; inverse of chunk 0.
#   recurrence w, step s >= 0: wait until every rdone >= s + 5 and gready of
#     group s == s + 6; read the record of chunk s and the value rows of group
#     s; inverse of chunk s + 1.
# ---------------------------------------------------------------------------

def simulate_fused(D, nch, seed, drop=None, explicit=False):
    """explicit: the recurrence waves also wait for the record of chunk s
    (pdone[s mod 4] >= s + 4) and for L of chunk s + 1 (pdone[(s + 1) mod 4]
    >= s + 5).  The kernel leaves both out: the prep wave that finishes chunk
    s + 1 (phase 3, step s - 1) is the one that loads group s and reports it
    only at the top of step s, so the group wait implies the second, and the
    previous step's group wait (or, at s = 0, the wait before the inverse of
    chunk 0) implies the first."""
    rnd = random.Random(seed)
    R = 4
    grp = {}                       # slot -> [group, landed]
    grp_users = {}                 # slot -> set of pending readers of its group
    rec = {}                       # slot -> dict(chunk, phases done, T parts)
    rec_users = {}                 # slot -> set of pending readers of its chunk
    lts = {}                       # buffer -> (chunk, complete)
    lts_users = {}
    reading = []                   # (kind, slot) being read right now, with owner
    pdone = [0] * 4
    rdone = [4] * R
    gready = [0] * D
    in_flight = {}                 # prep wave -> group it has in flight

    def gslot(g):
        return (g + 5) % D

    def start_group(g, owner):
        sl = gslot(g)
        if grp_users.get(sl):
            raise AssertionError("group %d overwrites slot %d still needed for group %s" % (g, sl, grp[sl][0]))
        if any(k == "grp" and x == sl for k, x, _ in reading):
            raise AssertionError("group slot %d overwritten while read" % sl)
        grp[sl] = [g, False]
        users = set()
        if g + 5 < nch:                # phase 0 of chunk g + 5 reads its raw inputs
            users.add(("prep", (g + 5) % 4))
        if 0 <= g < nch:               # step g reads its value rows
            users |= {("rec", w) for w in range(R)}
        grp_users[sl] = users
        in_flight[owner] = g

    def land(owner):
        g = in_flight.pop(owner)
        grp[gslot(g)][1] = True

    prep = [{"s": -5, "stage": "top", "left": 0} for _ in range(4)]
    recw = [{"s": -1, "stage": "wait", "left": 0} for _ in range(R)]
    # prologue groups
    for g in range(-5, min(-5 + D - 1, nch)):
        start_group(g, (g + 5) % 4)
        if rnd.random() < 0.5:
            land((g + 5) % 4)

    def rec_min():
        return min(rdone)

    for _ in range(3_000_000):
        actors = [("P", p) for p in range(4) if prep[p]["s"] < nch]
        actors += [("R", w) for w in range(R) if recw[w]["s"] < nch]
        if not actors and not in_flight:
            return
        if in_flight and rnd.random() < 0.25:      # some load lands
            land(rnd.choice(list(in_flight)))
            continue
        if not actors:
            continue
        kind, i = rnd.choice(actors)
        if kind == "P":
            st = prep[i]
            s = st["s"]
            if st["stage"] == "top":
                if ((s + 5) & 3) == i:             # its own group s: vmcnt(0)
                    if i in in_flight:
                        continue
                    if drop != "gready":
                        gready[gslot(s)] = s + 6
                st["stage"] = "wait"
            elif st["stage"] == "wait":
                need = s + 5 - (1 if drop == "prep_rec" else 0)
                if rec_min() < need:
                    continue
                g = s + D - 1
                if g < nch and ((g + 5) & 3) == i:
                    if drop != "prep_issue" and pdone[(s + 4) & 3] < s + 5:
                        continue
                    if i in in_flight:
                        raise AssertionError("two groups in flight on one prep wave")
                    start_group(g, i)
                ph = (s + 5 - i) & 3
                c = s + 5 - ph
                st["work"] = None
                if 0 <= c < nch:
                    sl = c % 6
                    if ph == 0:
                        gs = gslot(s)
                        if grp.get(gs) != [s, True]:
                            raise AssertionError("phase 0 of chunk %d reads group slot without group %d" % (c, s))
                        if rec_users.get(sl):
                            raise AssertionError("chunk %d overwrites record slot %d still needed" % (c, sl))
                        if any(k == "rec" and x == sl for k, x, _ in reading):
                            raise AssertionError("record slot %d overwritten while read" % sl)
                        rec[sl] = {"c": c, "ph": 0, "T": set()}
                        rec_users[sl] = {("rec", w) for w in range(R)} | {("inv", w) for w in range(R)}
                        reading.append(("grp", gs, ("P", i)))
                    else:
                        if rec[sl]["c"] != c or rec[sl]["ph"] != ph:
                            raise AssertionError("phase order broken for chunk %d" % c)
                    if ph == 3:
                        b = c & 1
                        if lts_users.get(b):
                            raise AssertionError("L of chunk %d overwrites a buffer still needed" % c)
                        lts[b] = (c, False)
                        lts_users[b] = {("inv", w) for w in range(R)}
                    st["work"] = (c, ph, sl)
                st["stage"] = "work"
                st["left"] = rnd.randint(1, 4)
            else:
                st["left"] -= 1
                if st["left"] > 0:
                    continue
                if st["work"] is not None:
                    c, ph, sl = st["work"]
                    if ph == 0:
                        reading.remove(("grp", gslot(s), ("P", i)))
                        grp_users[gslot(s)].discard(("prep", i))
                    rec[sl]["ph"] = ph + 1
                    if ph == 3:
                        lts[c & 1] = (c, True)
                pdone[i] = s + 6
                st["s"] = s + 1
                st["stage"] = "top"
        else:
            st = recw[i]
            s = st["s"]
            if st["stage"] == "wait":
                if s == -1:
                    if pdone[0] < 4:
                        continue
                else:
                    if explicit and pdone[s & 3] < s + 4:
                        continue
                    if explicit and pdone[(s + 1) & 3] < s + 5:
                        continue
                    if drop != "rec_T" and rec_min() < s + 5:
                        continue
                    if drop != "rec_group" and gready[gslot(s)] != s + 6:
                        continue
                    sl = s % 6
                    r = rec.get(sl)
                    if r is None or r["c"] != s or r["ph"] != 4 or len(r["T"]) != R:
                        raise AssertionError("step %d reads an incomplete record %s" % (s, r))
                    if grp.get(gslot(s)) != [s, True]:
                        raise AssertionError("step %d reads value rows not landed" % s)
                    reading.append(("rec", sl, ("R", i)))
                    reading.append(("grp", gslot(s), ("R", i)))
                n = s + 1                      # the inverse of chunk n
                if n < nch:
                    b = n & 1
                    if lts.get(b) != (n, True):
                        raise AssertionError("inverse of chunk %d reads an incomplete L" % n)
                    r = rec.get(n % 6)
                    if r is None or r["c"] != n or r["ph"] < 1:
                        raise AssertionError("inverse of chunk %d without its beta" % n)
                st["stage"] = "work"
                st["left"] = rnd.randint(1, 4)
            else:
                st["left"] -= 1
                if st["left"] > 0:
                    continue
                if s >= 0:
                    reading.remove(("rec", s % 6, ("R", i)))
                    reading.remove(("grp", gslot(s), ("R", i)))
                    rec_users[s % 6].discard(("rec", i))
                    grp_users[gslot(s)].discard(("rec", i))
                n = s + 1
                if n < nch:
                    rec[n % 6]["T"].add(i)
                    rec_users[n % 6].discard(("inv", i))
                    lts_users[n & 1].discard(("inv", i))
                rdone[i] = s + 6
                st["s"] = s + 1
                st["stage"] = "wait"
    raise AssertionError("no progress: the waves deadlocked")


@pytest.mark.parametrize("explicit", [False, True])
@pytest.mark.parametrize("D", [3, 4, 5])
def test_fused_flag_protocol_is_safe_and_live(D, explicit):
    for nch in (1, 2, 3, 4, 5, 7, 8, 13, 20):
        for seed in range(6):
            simulate_fused(D, nch, seed, explicit=explicit)


@pytest.mark.parametrize("drop", ["prep_rec", "prep_issue", "rec_T", "rec_group", "gready"])
def test_fused_dropped_wait_is_caught(drop):
    with pytest.raises(AssertionError, match="reads|overwrite|needed|deadlock|landed|incomplete|without"):
        for seed in range(300):
            for D in (3, 4):
                simulate_fused(D, 13, seed, drop=drop)
