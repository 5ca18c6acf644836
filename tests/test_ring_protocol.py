"""The barrier ring of the pipelined kernel, model-checked on the CPU for every copy mode.

The model restates, per copy mode (staging 0, 1, 4, 5, 6, 7), the sequence of events one
wave of pipelined_gemm runs: copies into LDS slots (direct-to-LDS copies that land later,
in issue order; or, for the register-staged modes, loads into registers and LDS writes
from them), `s_waitcnt vmcnt(N)` waits, fragment reads of a k-tile's slot, and the
workgroup barrier (preceded by `s_waitcnt lgkmcnt(0)`, so a wave's LDS reads and writes
are complete when it arrives).  Every wave runs the same program and waves meet only at
barriers, so barrier generations decide what is safe:

  * read after write: a fragment read of k-tile t from a slot happens in a generation
    at or after the one in which every copy of t into that slot was published (the
    copying wave waited for it, then passed a barrier);
  * write after read: no copy or LDS write into a slot is issued in a generation in which
    any wave may still be reading the k-tile the slot held (reads of generation g are
    complete only at barrier g + 1);
  * register staging writes, into a slot, the k-tile that slot is meant to receive;
  * the epilogue, which reuses the ring for staging, starts after every copy has landed
    and every read is complete.

The premature slot reuse the Pallas guide warns about (delay_release) is exactly a
write-after-read failure here; planted variants (one k-tile too few waited for, a refill
issued before the barrier that releases the slot) are caught.
"""

import pytest


class Violation(AssertionError):
    pass


class Ring:
    """LDS contents and the hazard checks.  A 'part' is one operand's array in a slot."""

    def __init__(self, n_ops_a, n_ops_b):
        self.na, self.nb = n_ops_a, n_ops_b
        self.gen = 0                 # barriers passed
        self.holder = {}             # part -> k-tile it holds
        self.published = {}          # part -> {op: generation it became visible}
        self.last_read = {}          # part -> (k-tile, generation of the last read)
        self.pending = []            # direct copies in flight, issue order: (part, kt, op)
        self.regs = {}               # register staging: op -> k-tile loaded

    def _write(self, part, kt, op):
        old = self.last_read.get(part)
        if old is not None and old[0] != kt and old[1] >= self.gen:
            raise Violation(f"{part} refilled with k-tile {kt} in generation {self.gen} while "
                            f"k-tile {old[0]} may still be read (read in generation {old[1]})")
        if self.holder.get(part) != kt:
            self.holder[part] = kt
            self.published[part] = {}
        self.published[part][op] = None      # not visible yet

    def copy(self, part, kt, op):
        """A direct-to-LDS copy: issued now, lands later (in issue order)."""
        self._write(part, kt, op)
        self.pending.append((part, kt, op))

    def wait_vmcnt(self, n):
        while len(self.pending) > n:
            part, kt, op = self.pending.pop(0)
            if self.holder.get(part) == kt:
                self.published[part][op] = "landed"

    def load(self, op, kt):
        self.regs[op] = kt

    def lwrite(self, part, kt, j, op):
        """A register-staged LDS write of copy op j (op `op` of its operand part) for
        k-tile kt, from the registers that op j loaded."""
        if self.regs.get(j) != kt:
            raise Violation(f"LDS write of k-tile {kt} op {j} from registers holding "
                            f"k-tile {self.regs.get(j)}")
        self._write(part, kt, op)
        self.published[part][op] = "landed"   # complete at the next lgkmcnt(0)

    def barrier(self):
        self.gen += 1
        for part, ops in self.published.items():
            for op, st in ops.items():
                if st == "landed":
                    ops[op] = self.gen

    def read(self, part, kt, nops):
        if self.holder.get(part) != kt:
            raise Violation(f"k-tile {kt} read from {part}, which holds {self.holder.get(part)}")
        ops = self.published[part]
        for op in range(nops):
            g = ops.get(op)
            if g is None or g == "landed" or g > self.gen:
                raise Violation(f"k-tile {kt} read from {part} in generation {self.gen} before "
                                f"copy op {op} was published")
        self.last_read[part] = (kt, self.gen)

    def epilogue(self):
        if self.pending:
            raise Violation("epilogue reuses the ring with copies still in flight")
        self.barrier()


def run_kernel(ldm, S, nk, ksteps, pf, na, nb, mutate=None):
    """One wave's program for copy mode `ldm`, as pipelined_gemm issues it."""
    L = na + nb
    r = Ring(na, nb)
    direct = ldm in (0, 4, 5, 6)
    reg = ldm in (1, 7)
    deep = ldm in (4, 6)

    def slot_of(i):
        return (f"r{i}.A", f"r{i}.B")

    def deep_slot(i):
        if ldm == 6:
            return (f"r{i % 2}.A", ("r0.B", "r1.B", "b2")[i % 3])
        return (("r0.A", "r1.A", "a2")[i % 3], f"r{i % 2}.B")

    def slot_at(t):
        return deep_slot(t % 6) if deep else slot_of(t % S)

    def ops_order():
        # the A-deep ring copies B before A; the others A (ops 0 .. na-1) then B
        return list(range(na, L)) + list(range(na)) if ldm == 4 else list(range(L))

    def issue(slot, kt_a, kt_b, ops=None):
        for j in ops if ops is not None else ops_order():
            if j < na:
                r.copy(slot[0], kt_a, j)
            else:
                r.copy(slot[1], kt_b, j - na)

    def read_step(slot, kt):
        r.read(slot[0], kt, na)
        r.read(slot[1], kt, nb)

    # --- prologue ---
    if ldm == 0:
        for s in range(S):
            issue(slot_of(s), s, s)
        r.wait_vmcnt((S - 1) * L)
    elif ldm == 4:
        issue(deep_slot(0), 0, 0)
        issue(deep_slot(1), 1, 1)
        issue(deep_slot(2), 2, 2, ops=list(range(na)))
        r.wait_vmcnt(L + na)
    elif ldm == 6:
        issue(deep_slot(0), 0, 0)
        issue(deep_slot(1), 1, 1)
        issue(deep_slot(2), 2, 2, ops=list(range(na, L)))
        r.wait_vmcnt(L + nb)
    elif ldm == 5:
        for s in range(S - 1):
            issue(slot_of(s), s, s)
        r.wait_vmcnt((S - 2) * L)
    else:
        cps = L // ksteps
        pre = pf * cps
        for s in range(S - 1):
            for j in range(L):
                r.load(j, s)
            for j in range(L):
                part = slot_of(s)[0 if j < na else 1]
                r.lwrite(part, s, j, j if j < na else j - na)
        for j in range(L):
            r.load(j, S - 1)
        for j in range(pre):
            r.lwrite(slot_of(S - 1)[0 if j < na else 1], S - 1, j, j if j < na else j - na)
            r.load(j, S)
    r.barrier()
    for _ in range(pf):
        read_step(slot_at(0), 0)

    steady = {4: na, 6: nb, 5: (S - 3) * L}.get(ldm, (S - 2) * L)
    if mutate == "wait_one_tile_less":
        steady += L

    def ktile(t):
        cur, prev, nxt = slot_at(t), slot_at(t - 1), slot_at(t + 1)
        # stages before the barrier: reads of the next steps (of k-tile t, then t+1)
        if reg:
            cps = L // ksteps
            for kk in range(ksteps - pf):
                j0 = (pf + kk) * cps
                for j in range(j0, j0 + cps):
                    r.lwrite(prev[0 if j < na else 1], t + S - 1, j, j if j < na else j - na)
                    r.load(j, t + S)
                rk = kk + pf
                read_step(cur if rk < ksteps else nxt, t if rk < ksteps else t + 1)
        else:
            if mutate == "refill_before_barrier":
                issue(cur, t + S, t + S)
            for kk in range(ksteps - pf):
                rk = kk + pf
                read_step(cur if rk < ksteps else nxt, t if rk < ksteps else t + 1)
            r.wait_vmcnt(steady)
        r.barrier()
        # stages after the barrier: the window's copies, reads of k-tile t+1
        if direct and mutate != "refill_before_barrier":
            if ldm == 4:
                issue(cur, t + 3, t + 2)
            elif ldm == 6:
                issue(cur, t + 2, t + 3)
            elif ldm == 5:
                issue(prev, t + S - 1, t + S - 1)
            else:
                issue(cur, t + S, t + S)
        if reg:
            cps = L // ksteps
            for kk in range(ksteps - pf, ksteps):
                j0 = (kk - (ksteps - pf)) * cps
                for j in range(j0, j0 + cps):
                    r.lwrite(cur[0 if j < na else 1], t + S, j, j if j < na else j - na)
                    r.load(j, t + S + 1)
        for kk in range(ksteps - pf, ksteps):
            rk = kk + pf
            read_step(cur if rk < ksteps else nxt, t if rk < ksteps else t + 1)

    if deep:
        t0 = 0
        while t0 + 6 <= nk:
            for s in range(6):
                ktile(t0 + s)
            t0 += 6
        for s in range(nk - t0):
            ktile(t0 + s)
    else:
        nt = ((nk + S - 1) // S) * S
        for t in range(nt):
            ktile(t)
    if mutate != "no_final_wait":
        r.wait_vmcnt(0)
    r.epilogue()
    return r.gen


# (mode, stages, k-steps per k-tile, lookahead, copy ops of A and B per wave) as compiled:
# 8 waves of 256x256x64 (16x16x32: 2 k-steps; 32x32x16: 4), 4 waves of 128x128x64,
# BK = 32 rings, register staging, the deep rings
CONFIGS = [(0, 2, 2, 1, 4, 4), (0, 2, 4, 1, 4, 4), (0, 3, 4, 1, 4, 4), (0, 4, 4, 1, 4, 4),
           (0, 2, 4, 2, 8, 8), (0, 4, 2, 1, 4, 4), (0, 5, 2, 1, 4, 4), (0, 3, 2, 1, 4, 2),
           (1, 2, 4, 1, 8, 8), (1, 3, 2, 1, 4, 4), (1, 2, 4, 2, 8, 8), (1, 3, 4, 1, 4, 4),
           (7, 2, 4, 1, 4, 4), (7, 3, 4, 1, 8, 4), (7, 3, 4, 1, 4, 4),
           (4, 2, 4, 1, 4, 4), (6, 2, 2, 1, 4, 4),
           (5, 3, 4, 1, 4, 4), (5, 3, 4, 1, 4, 2)]


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "ldm{}_S{}_k{}_pf{}_{}x{}".format(*c))
def test_ring_is_race_free(cfg):
    ldm, S, ksteps, pf, na, nb = cfg
    for nk in range(1, 20):
        run_kernel(ldm, S, nk, ksteps, pf, na, nb)


@pytest.mark.parametrize("mutate,ldm", [("wait_one_tile_less", 0), ("wait_one_tile_less", 6),
                                        ("wait_one_tile_less", 4), ("refill_before_barrier", 0),
                                        ("refill_before_barrier", 5), ("no_final_wait", 0)])
def test_model_catches_planted_mistakes(mutate, ldm):
    S = {0: 2, 4: 2, 5: 3, 6: 2}[ldm]
    ksteps = 2 if ldm == 6 else 4
    with pytest.raises(Violation):
        for nk in range(1, 20):
            run_kernel(ldm, S, nk, ksteps, 1, 4, 4, mutate=mutate)


def test_register_staging_mismatch_is_caught():
    # staging that wrote the k-tile loaded one window too early would write the wrong data
    r = Ring(2, 2)
    r.load(0, 5)
    with pytest.raises(Violation):
        r.lwrite("r0.A", 4, 0, 0)
