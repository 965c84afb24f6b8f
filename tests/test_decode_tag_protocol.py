"""Host-side model of the decode path's cross-workgroup handoff (two to four
rows): router waves publish each logit in a 64-bit word {call tag, value};
the plan block polls its rows' words until all carry the call's tag, routes,
and (since the fix) sets every word it consumed back to 0.

The model replays, on the CPU, every interleaving of the operations a caller
can issue on one workspace -- eager calls of 1, 2 and 4 rows, prefill calls,
capturing a graph of one or two 2-4-row calls, replaying captured graphs --
and checks the property the plan block relies on: when a call starts, no
word of its rows already carries its tag (otherwise the poll could accept a
word before this call's router has written it).

Tag of a call = host value (a process-wide counter, frozen into a captured
graph) + the workspace's device call count (advanced once per 2-4-row call);
a tag of 0 becomes 1.  One-row and prefill calls touch neither the words nor
the count.  The workspace starts zero-filled (the ABI's contract).
"""

from __future__ import annotations

import itertools

import pytest

MASK32 = (1 << 32) - 1


class Workspace:
    def __init__(self, call_seq=0, rows=4, experts=3):
        self.call_seq = call_seq & MASK32
        self.words = {(r, e): 0 for r in range(rows) for e in range(experts)}
        self.experts = experts


class Host:
    """The library's process-wide host counter (never hands out 0)."""

    def __init__(self, start):
        self.ctr = start & MASK32

    def next_epoch(self):
        e = self.ctr
        self.ctr = (self.ctr + 1) & MASK32
        if e == 0:
            e = self.ctr
            self.ctr = (self.ctr + 1) & MASK32
        return e


def run_call(ws: Workspace, rows: int, epoch: int, clear: bool, value: int) -> bool:
    """One forward of `rows` rows with host value `epoch`; returns False if a
    word of the call's rows carried the call's tag before its router wrote."""
    if rows == 1 or rows > 4:
        return True  # the one-row path and prefill use no tagged words
    tag = (epoch + ws.call_seq) & MASK32
    tag = tag or 1
    ok = all((ws.words[(r, e)] >> 32) != tag for r in range(rows) for e in range(ws.experts))
    for r in range(rows):  # router waves
        for e in range(ws.experts):
            ws.words[(r, e)] = (tag << 32) | (value & MASK32)
    if clear:  # plan block: consumed words back to 0
        for r in range(rows):
            for e in range(ws.experts):
                ws.words[(r, e)] = 0
    ws.call_seq = (ws.call_seq + 1) & MASK32  # gate/up launch
    return ok


def run_sequence(ops, clear, host_start, seq_start):
    """Apply `ops` to one workspace; returns the index of the first op whose
    call could read a stale word, or None."""
    ws = Workspace(seq_start)
    host = Host(host_start)
    graphs = []
    val = 0
    for i, op in enumerate(ops):
        kind = op[0]
        calls = []
        if kind == "eager":
            calls = [(op[1], host.next_epoch())]
        elif kind == "capture":  # recording enqueues nothing; the host values freeze
            graphs.append([(r, host.next_epoch()) for r in op[1]])
        elif kind == "replay":
            if not graphs:
                continue
            calls = graphs[op[1] % len(graphs)]
        for rows, ep in calls:
            val += 1
            if not run_call(ws, rows, ep, clear, val):
                return i
    return None


OPS = [("eager", 4), ("eager", 2), ("eager", 1), ("eager", 64), ("capture", (4, 4)), ("capture", (4,)),
       ("capture", (2, 1, 3)), ("replay", 0), ("replay", 1)]
STARTS = [(1, 0), (7, 5), (MASK32 - 2, 0), (0x9e3779b9, MASK32 - 1), (MASK32, MASK32)]


def test_old_protocol_collides_on_two_layer_graph_replays():
    """Without the reset, two 4-row calls captured in one graph on one
    workspace collide on the second replay: layer 0 of replay r+1 gets the
    tag layer 1 used in replay r (host h vs h+1, device count s+2 vs s+1)."""
    ops = [("capture", (4, 4)), ("replay", 0), ("replay", 0)]
    assert run_sequence(ops, clear=False, host_start=100, seq_start=0) == 2
    assert run_sequence(ops, clear=True, host_start=100, seq_start=0) is None
    # an eager call whose host value is one below a captured call's collides
    # with that call's next replay: eager h then replay h+1 after one call
    ops = [("eager", 4), ("capture", (4,)), ("replay", 0), ("eager", 4), ("replay", 0)]
    assert run_sequence(ops, clear=False, host_start=100, seq_start=0) is not None
    assert run_sequence(ops, clear=True, host_start=100, seq_start=0) is None


@pytest.mark.parametrize("host_start,seq_start", STARTS)
def test_reset_protocol_never_reads_a_stale_word(host_start, seq_start):
    """Every sequence of up to 5 operations (9^5 = 59049 of them, each from
    five starting states including counter wrap-around) is safe once the
    plan block sets consumed words back to 0."""
    bad = 0
    for n in range(1, 6):
        for ops in itertools.product(OPS, repeat=n):
            if run_sequence(ops, clear=True, host_start=host_start, seq_start=seq_start) is not None:
                bad += 1
    assert bad == 0


def test_old_protocol_fails_somewhere_in_the_same_enumeration():
    """The enumeration is strong enough to see the bug: without the reset,
    some of the same sequences read a stale word."""
    bad = 0
    for ops in itertools.product(OPS, repeat=3):
        if run_sequence(ops, clear=False, host_start=100, seq_start=0) is not None:
            bad += 1
    assert bad > 0
