"""The wave-specialized ring's counter protocol (ws_gemm, staging 3), model-checked on the CPU.

A model of one workgroup: a producer wave and NC consumer waves step through the same
sequence the kernel runs, with the same counter arithmetic, under random interleavings;
copies complete at random later times, in issue order (s_waitcnt vmcnt semantics).
Checked on every run:
  * no deadlock: until everyone is done some wave can always move;
  * no slot is refilled while a consumer can still read the k-tile it held;
  * no consumer reads a k-tile before all of its copies have landed.
The model is the protocol, not the kernel: it pins the design (counters, targets, the
order of the release and the wait), which GPU parity alone cannot show to be race-free.
"""

import random

import pytest


def run_protocol(nk, S, NC, rng, short=0, max_steps=1_000_000):
    """short: releases per reuse the producer does not wait for (0 = the kernel's protocol)."""
    full = [0] * S          # 1 + last k-tile completed into slot s
    freed = [0] * S         # consumer releases of slot s
    holder = [None] * S     # k-tile the slot's contents belong to (None: empty)
    landed = set()          # k-tiles whose copies have all completed
    in_flight = []          # k-tiles issued, not yet landed (completes in order)
    reading = {}            # (consumer) -> k-tile whose slot it may read
    # producer program counter: ("issue", t) / ("wait_vmcnt", t) / ("publish", t) / done
    prod = {"t": 0, "phase": "issue0"}
    cons = [{"t": 0, "phase": "wait_first"} for _ in range(NC)]

    def slot_writable(t):
        s = t % S
        return holder[s] is None or all(r != holder[s] for r in reading.values())

    def producer_step():
        p = prod
        if p["phase"] == "issue0":
            assert slot_writable(0)
            holder[0] = 0; in_flight.append(0); p["t"] = 1
            p["phase"] = "loop" if nk > 1 else "drain"
            return True
        if p["phase"] == "loop":
            t = p["t"]
            if t >= S and freed[t % S] < (NC - short) * (t // S):
                return False                      # waits on freed
            assert slot_writable(t), f"slot {t % S} refilled while k-tile {holder[t % S]} is read"
            holder[t % S] = t; in_flight.append(t)
            p["phase"] = "wait_prev"
            return True
        if p["phase"] == "wait_prev":             # s_waitcnt vmcnt(L): k-tile t-1 landed
            t = p["t"]
            if (t - 1) not in landed:
                return False
            full[(t - 1) % S] = t                 # publish t-1
            p["t"] = t + 1
            p["phase"] = "loop" if t + 1 < nk else "drain"
            return True
        if p["phase"] == "drain":                 # s_waitcnt vmcnt(0); publish nk-1
            if (nk - 1) not in landed:
                return False
            full[(nk - 1) % S] = nk
            p["phase"] = "done"
            return True
        return False

    def consumer_step(i):
        c = cons[i]
        if c["phase"] == "wait_first":
            if full[0] < 1:
                return False
            reading[i] = 0
            c["phase"] = "compute"
            return True
        t = c["t"]
        if c["phase"] == "compute":               # reads of k-tile t (steps 1..3)
            assert t in landed, f"k-tile {t} read before its copies landed"
            assert holder[t % S] == t, f"slot {t % S} refilled while k-tile {t} is read"
            c["phase"] = "release"
            return True
        if c["phase"] == "release":               # lgkmcnt(0), freed[t % S] += 1
            freed[t % S] += 1
            reading.pop(i, None)
            c["phase"] = "wait_next" if t + 1 < nk else "done"
            return True
        if c["phase"] == "wait_next":             # wait full[(t+1) % S] >= t + 2
            if full[(t + 1) % S] < t + 2:
                return False
            reading[i] = t + 1                    # reads step 0 of k-tile t+1
            assert (t + 1) in landed, f"k-tile {t + 1} read before its copies landed"
            assert holder[(t + 1) % S] == t + 1, f"slot {(t + 1) % S} refilled while k-tile {t + 1} is read"
            c["t"] = t + 1
            c["phase"] = "compute"
            return True
        return False

    def complete_copy():
        if in_flight:
            landed.add(in_flight.pop(0))
            return True
        return False

    for _ in range(max_steps):
        if prod["phase"] == "done" and all(c["phase"] == "done" for c in cons):
            return True
        actors = [producer_step] + [lambda i=i: consumer_step(i) for i in range(NC)] + [complete_copy]
        rng.shuffle(actors)
        if not any(a() for a in actors[:1]) and not any(a() for a in actors[1:]):
            raise AssertionError("deadlock: no wave can move")
    raise AssertionError("did not finish")


@pytest.mark.parametrize("S", [2, 3, 4])
@pytest.mark.parametrize("nk", [1, 2, 3, 5, 17])
def test_protocol_random_interleavings(S, nk):
    rng = random.Random(1000 * S + nk)
    for _ in range(300):
        assert run_protocol(nk, S, 4, rng)


def test_protocol_check_is_live():
    # a producer that waits for one consumer release fewer than it must refills a slot
    # that is still being read in some interleaving: the model catches it
    rng = random.Random(7)
    caught = 0
    for _ in range(300):
        try:
            run_protocol(6, 2, 4, rng, short=1)
        except AssertionError as e:
            assert "refilled" in str(e)
            caught += 1
    assert caught > 0
