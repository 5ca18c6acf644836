"""The ping-pong schedule's ring protocol, model-checked on the CPU.

In the ping-pong schedule (schedule 2, B-deep ring) the waves of a workgroup form two
groups that run different programs: group 1 passes one extra barrier before its first
phase and group 0 one after its last, so between any two workgroup barriers one group is
in a memory phase (fragment reads of one k-step, and in the first k-step of a k-tile its
copies into the slots the previous k-tile released) while the other is in a matrix phase
(MFMAs only).  The model restates both programs as the kernel issues them and runs them
phase by phase, a phase being the span between two consecutive barriers:

  * each group has its own queue of direct-to-LDS copies, which land in issue order;
    `s_waitcnt vmcnt(N)` in phase p lands all but the last N of them, and the barrier at
    the end of phase p makes them visible from phase p+1 on;
  * a memory phase ends with `s_waitcnt lgkmcnt(0)`, so its reads are complete at the
    barrier that ends it;
  * read after write: a read of k-tile t from a slot part in phase p needs every copy op
    of t into that part, from both groups, landed in a phase before p;
  * write after read: a copy into a part in phase p needs every read of the k-tile the
    part held, by both groups, to lie in a phase before p;
  * the epilogue (the ring reused for staging) starts after both groups' copies have
    landed and both have passed the same number of barriers.

Planted variants of the protocol (group 1's wait one phase late, a wait for one k-tile
too few, a refill one k-tile early into the slot being read) must be caught.  Two variants
that are safe are shown to be safe: the copies moved to the second memory phase of a
k-tile (less lead, no hazard) and the two groups in lockstep (no turns, no hazard).
"""

import pytest


class Violation(AssertionError):
    pass


def programs(nk, na, nb, mutate=None):
    """The two groups' programs: lists of phases, each a list of actions.  Actions:
    ("copy", part, kt, op), ("wait", n), ("read", part, kt).  Slots of the B-deep ring:
    A parts t % 2, B parts t % 3; copy ops 0 .. na-1 move A, na .. na+nb-1 move B, and
    each group issues its own ops (op ids are (group, j))."""
    L = na + nb

    def a_part(t):
        return f"A{t % 2}"

    def b_part(t):
        return f"B{t % 3}"

    progs = []
    for grp in (0, 1):
        phases = []
        # prologue: k-tiles 0 and 1, and B of k-tile 2; wait for k-tile 0; barrier
        pro = []
        for t in (0, 1):
            pro += [("copy", a_part(t), t, (grp, j)) for j in range(na)]
            pro += [("copy", b_part(t), t, (grp, na + j)) for j in range(nb)]
        pro += [("copy", b_part(2), 2, (grp, na + j)) for j in range(nb)]
        pro += [("wait", L + nb)]
        phases.append(pro)
        if grp == 1 and mutate != "no_offset":
            phases.append([])          # one phase behind group 0
        late_wait = mutate == "group1_waits_late"
        for u in range(nk):
            m0 = [("read", a_part(u), u), ("read", b_part(u), u)]
            copies = []
            if u >= 1:
                e = 1 if mutate == "refill_early" else 0
                copies += [("copy", a_part(u + 1 + e), u + 1 + e, (grp, j)) for j in range(na)]
                copies += [("copy", b_part(u + 2 + e), u + 2 + e, (grp, na + j)) for j in range(nb)]
            steady = nb + (L if mutate == "one_tile_less" else 0)
            if mutate == "copies_in_second_step":
                m1 = [("read", a_part(u), u), ("read", b_part(u), u)] + copies
                m0_full = m0
            else:
                m1 = [("read", a_part(u), u), ("read", b_part(u), u)]
                m0_full = m0 + copies
            c0 = []
            c1 = []
            if grp == 1 and not late_wait:
                m1 = m1 + [("wait", steady)]
            else:
                c1 = [("wait", steady)]
            phases += [m0_full, c0, m1, c1]
        if grp == 0 and mutate != "no_offset":
            phases.append([])          # matches group 1's extra barrier
        # epilogue: all copies landed before the ring is reused
        phases.append([("wait", 0)])
        progs.append(phases)
    return progs


def check(progs, na, nb):
    n_phases = {len(p) for p in progs}
    if len(n_phases) != 1:
        raise Violation(f"the groups pass different numbers of barriers: {n_phases}")
    n = n_phases.pop()
    pending = [[], []]                 # per group: (part, kt, op) in issue order
    landed = {}                        # (part, kt, op) -> phase it landed in
    holder = {}                        # part -> k-tile it is being filled with / holds
    last_read = {}                     # (part, kt) -> last phase it was read in
    for p in range(n):
        acts = [progs[g][p] for g in (0, 1)]
        # reads first (a read and a copy of the same part in one phase conflict either way)
        for g in (0, 1):
            for a in acts[g]:
                if a[0] != "read":
                    continue
                _, part, kt = a
                if holder.get(part) != kt:
                    raise Violation(f"phase {p}: group {g} reads k-tile {kt} from {part}, "
                                    f"which holds {holder.get(part)}")
                ops = [(h, j) for h in (0, 1)
                       for j in (range(na) if part[0] == "A" else range(na, na + nb))]
                for op in ops:
                    ph = landed.get((part, kt, op))
                    if ph is None or ph >= p:
                        raise Violation(f"phase {p}: group {g} reads k-tile {kt} from {part} "
                                        f"before copy op {op} was published")
                last_read[(part, kt)] = p
        for g in (0, 1):
            for a in acts[g]:
                if a[0] == "copy":
                    _, part, kt, op = a
                    old = holder.get(part)
                    if old is not None and old != kt:
                        lr = last_read.get((part, old))
                        if lr is not None and lr >= p:
                            raise Violation(f"phase {p}: group {g} refills {part} with k-tile "
                                            f"{kt} while k-tile {old} is read in phase {lr}")
                    holder[part] = kt
                    pending[g].append((part, kt, op))
                elif a[0] == "wait":
                    while len(pending[g]) > a[1]:
                        landed[pending[g].pop(0)] = p
    if pending[0] or pending[1]:
        raise Violation("copies still in flight at the epilogue")
    return n


@pytest.mark.parametrize("nk", list(range(1, 21)))
def test_ping_pong_is_race_free(nk):
    # the kernel's copy ops per wave with 8 waves on 256x256x64: 4 of A and 4 of B; the
    # model takes a group's share as one stream (each wave waits for its own copies, and
    # the group's waits are the same instruction in each of its waves)
    check(programs(nk, 4, 4), 4, 4)


def test_every_k_tile_is_read_by_both_groups_in_turn():
    # the offset holds: in every phase after the prologue at most one group reads
    progs = programs(7, 4, 4)
    n = check(progs, 4, 4)
    for p in range(1, n):
        readers = [g for g in (0, 1) if any(a[0] == "read" for a in progs[g][p])]
        assert len(readers) <= 1, (p, readers)


@pytest.mark.parametrize("mutate", ["group1_waits_late", "one_tile_less", "refill_early"])
def test_model_catches_planted_mistakes(mutate):
    with pytest.raises(Violation):
        for nk in range(1, 12):
            check(programs(nk, 4, 4, mutate=mutate), 4, 4)


def test_copies_in_the_second_memory_phase_are_safe():
    # the refill issued one k-step later still lands before k-tile u+1 is read (group 1
    # issues and waits in the same memory phase): a shorter lead, not a hazard
    for nk in range(1, 12):
        check(programs(nk, 4, 4, mutate="copies_in_second_step"), 4, 4)


def test_groups_in_lockstep_lose_the_turns():
    # without the offset both groups read in the same phases: still race-free (the same
    # waits and barriers), but no phase pairs a matrix wave with a memory wave
    progs = programs(5, 4, 4, mutate="no_offset")
    n = check(progs, 4, 4)
    both = [p for p in range(1, n) if all(any(a[0] == "read" for a in progs[g][p]) for g in (0, 1))]
    assert both
