"""A CPU model of the persistent decode kernel's work queues: claim order,
residency and progress.

The model follows the kernel item for item.  Queue q (one per XCD) lists, in
this order:
  D(t, h)   for tokens t = q, q+8, ..., parts h < dpt             (none)
  F1(a, u)  for active experts a = q, q+8, ..., items u < upe1    needs every queue's D
  Q(a)      for the same experts                                  needs F1(a, *)
  F2(a, u)  items u < upe2                                        needs Q(a)
  C(t)      for the queue's tokens                                needs every queue's F2
and hands its items out by one ticket counter.  Before its first F1 item a
workgroup also takes part in the per-XCD invalidate: the first one of its
queue past the D wait claims it (mark 0 -> 1), invalidates, and sets the
mark to 2 (two steps in which it waits on nothing); the others wait for 2.  A workgroup serves the queue
of the XCD it runs on, so each queue has its own workgroups and its own
residency limit (an XCD runs at most so many of them at once; the others
start when a resident one exits).  A workgroup that holds an item whose
dependencies are unfinished waits (no progress); a workgroup exits when its
ticket is past the end of its queue.

The claim the kernel's progress rests on: every wait is for items of lower
order, so with at least one resident workgroup per queue, some workgroup can
always move, whatever the interleaving.  The tests run random interleavings
and residency limits and check that every item finishes; a planted mistake
(an item that waits on a later item of its own queue) must be caught.
"""
import random

import pytest

NQ = 8


def queue_items(q, T, n_act, upe1, upe2, c_before_f2=False, dpt=1):
    """The items of queue q in ticket order, as the kernel decodes tickets."""
    nD = (T - q + NQ - 1) // NQ if T > q else 0
    nA = (n_act - q + NQ - 1) // NQ if n_act > q else 0
    items = [("D", q + NQ * (i // dpt), i % dpt) for i in range(nD * dpt)]
    items += [("F1", q + NQ * (k // upe1), k % upe1) for k in range(nA * upe1)]
    items += [("Q", q + NQ * k) for k in range(nA)]
    f2 = [("F2", q + NQ * (k // upe2), k % upe2) for k in range(nA * upe2)]
    c = [("C", q + NQ * i) for i in range(nD)]
    items += (c + f2) if c_before_f2 else (f2 + c)
    return items


class Model:
    def __init__(self, T, n_act, upe1, upe2, wgs_per_queue, resident, c_before_f2=False, dpt=2,
                 mark_waits_for_expert=False):
        self.T, self.n_act, self.upe1, self.upe2 = T, n_act, upe1, upe2
        self.items = [queue_items(q, T, n_act, upe1, upe2, c_before_f2, dpt) for q in range(NQ)]
        self.nf2 = [sum(1 for it in self.items[q] if it[0] == "F2") for q in range(NQ)]
        self.nd = [sum(1 for it in self.items[q] if it[0] == "D") for q in range(NQ)]
        self.ticket = [0] * NQ
        self.d_q = [0] * NQ                       # D items done per queue
        self.d_queues = 0                         # queues whose D items are all done
        self.mark = [0] * NQ                      # per-XCD invalidate: 0 free, 1 claimed, 2 done
        self.mark_waits_for_expert = mark_waits_for_expert
        self.f1_done = [0] * n_act
        self.q_done = [False] * n_act
        self.f2_done = [0] * NQ
        self.queues_done = 0
        self.finished = 0
        self.total = sum(len(x) for x in self.items)
        # workgroups: per queue, the waiting-to-start count and the resident ones;
        # a resident one is [held item or None, token rows acquired, invalidate claimed]
        self.pending = list(wgs_per_queue)
        self.resident_cap = list(resident)
        self.res = [[] for _ in range(NQ)]
        for q in range(NQ):
            self._admit(q)

    def _admit(self, q):
        while self.pending[q] > 0 and len(self.res[q]) < self.resident_cap[q]:
            self.pending[q] -= 1
            self.res[q].append([None, False, False])

    def ready(self, it):
        kind = it[0]
        if kind == "D":
            return True
        if kind == "F1":
            return self.d_queues == min(self.T, NQ)
        if kind == "Q":
            return self.f1_done[it[1]] == self.upe1
        if kind == "F2":
            return self.q_done[it[1]]
        return self.queues_done == min(self.n_act, NQ)

    def can_act(self, q, wg):
        held, have_d, claimed = wg
        if held is None:
            return True                               # claims a ticket
        if not self.ready(held):
            return False
        if held[0] != "F1" or have_d:
            return True
        # first F1 item: the per-XCD invalidate
        if claimed and self.mark_waits_for_expert:    # planted mistake: the claimer waits on other items
            return self.f1_done[held[1]] >= self.upe1 - 1
        return claimed or self.mark[q] != 1

    def finish(self, q, it):
        kind = it[0]
        if kind == "D":
            self.d_q[q] += 1
            if self.d_q[q] == self.nd[q]:             # the increment that completes the queue's D items
                self.d_queues += 1
        elif kind == "F1":
            self.f1_done[it[1]] += 1
        elif kind == "Q":
            self.q_done[it[1]] = True
        elif kind == "F2":
            self.f2_done[q] += 1
            if self.f2_done[q] == self.nf2[q]:        # the increment that completes the queue
                self.queues_done += 1
        self.finished += 1

    def moves(self):
        """(queue, slot) of every resident workgroup that can act now."""
        return [(q, i) for q in range(NQ) for i, wg in enumerate(self.res[q]) if self.can_act(q, wg)]

    def step(self, q, i):
        wg = self.res[q][i]
        held = wg[0]
        if held is not None:
            if held[0] == "F1" and not wg[1]:         # first F1 item: the per-XCD invalidate first
                if wg[2]:                             # the claimer invalidates and sets the mark
                    self.mark[q] = 2
                    wg[1], wg[2] = True, False
                elif self.mark[q] == 0:               # first past the D wait: claim the invalidate
                    self.mark[q] = 1
                    wg[2] = True
                else:                                 # mark 2: invalidate this CU's L1
                    wg[1] = True
                return
            self.finish(q, held)                      # its dependencies are done: run it
            wg[0] = None
            return
        t = self.ticket[q]
        self.ticket[q] += 1
        if t >= len(self.items[q]):                  # past the end: the workgroup exits
            self.res[q].pop(i)
            self._admit(q)
        else:
            wg[0] = self.items[q][t]

    def run(self, rng, max_steps=10 ** 6):
        for _ in range(max_steps):
            if all(not r for r in self.res) and all(p == 0 for p in self.pending):
                return "done"
            mv = self.moves()
            if not mv:
                return "deadlock"
            self.step(*rng.choice(mv))
        return "too long"


@pytest.mark.parametrize("seed", range(40))
def test_every_item_finishes_for_any_interleaving_and_residency(seed):
    """Random batch shapes, unit counts, workgroups per queue (at least one)
    and residency limits (at least one per queue): every interleaving the
    random scheduler picks runs every item and lets every workgroup exit."""
    rng = random.Random(seed)
    T = rng.choice([0, 1, 3, 8, 9, 16, 37])
    n_act = rng.choice([0, 1, 5, 8, 13, 30]) if T else 0
    upe1, upe2 = rng.randint(1, 4), rng.randint(1, 5)
    wgs = [rng.randint(1, 6) for _ in range(NQ)]
    res = [rng.randint(1, w) for w in wgs]
    m = Model(T, n_act, upe1, upe2, wgs, res)
    assert m.run(rng) == "done", (T, n_act, upe1, upe2, wgs, res)
    assert m.finished == m.total
    assert m.d_queues == min(T, NQ) and m.queues_done == min(n_act, NQ)


def test_one_resident_workgroup_per_queue_is_enough():
    """The smallest residency the kernel needs: one workgroup per queue,
    resident alone; across several interleavings every item still finishes."""
    for seed in range(10):
        m = Model(16, 13, 3, 4, [1] * NQ, [1] * NQ)
        assert m.run(random.Random(seed)) == "done"


def test_planted_order_mistake_is_caught():
    """Negative check of the model: with C items listed before the F2 items
    of their own queue (a wait on a later item) and one resident workgroup
    per queue, some interleaving deadlocks, and the model reports it."""
    outcomes = set()
    for seed in range(20):
        m = Model(16, 13, 2, 2, [1] * NQ, [1] * NQ, c_before_f2=True)
        outcomes.add(m.run(random.Random(seed)))
    assert "deadlock" in outcomes


def test_planted_wait_in_the_invalidate_is_caught():
    """Negative check of the invalidate protocol's model: if the workgroup
    that claims a queue's invalidate waited for other F1 items of its expert
    before setting the mark (which those items' holders wait for), some
    interleaving deadlocks, and the model reports it."""
    outcomes = set()
    for seed in range(30):
        m = Model(16, 13, 4, 2, [3] * NQ, [3] * NQ, mark_waits_for_expert=True)
        outcomes.add(m.run(random.Random(seed)))
    assert "deadlock" in outcomes


def test_queue_items_cover_every_unit_once():
    """The per-queue ticket decode covers every token's D and C item and
    every expert's F1, Q and F2 units exactly once."""
    T, n_act, upe1, upe2 = 37, 30, 3, 5
    allit = [it for q in range(NQ) for it in queue_items(q, T, n_act, upe1, upe2)]
    assert len(allit) == len(set(allit))
    assert {it for it in allit if it[0] == "D"} == {("D", t, 0) for t in range(T)}
    assert {it for it in allit if it[0] == "C"} == {("C", t) for t in range(T)}
    assert {it for it in allit if it[0] == "F1"} == {("F1", a, u) for a in range(n_act) for u in range(upe1)}
    assert {it for it in allit if it[0] == "Q"} == {("Q", a) for a in range(n_act)}
    assert {it for it in allit if it[0] == "F2"} == {("F2", a, u) for a in range(n_act) for u in range(upe2)}
