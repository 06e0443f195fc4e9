"""Static race check of the default kernel's LDS ring (no GPU).

The persistent 4-wave kernel keeps five 32 KiB LDS slots: the A tile of the
step being computed at ring position sa, its B tile at sa + 1, the next
step's at sa + 2 and sa + 3, and the fifth slot filling with the A tile two
steps ahead.  A slot may be overwritten only after every wave has read what
it held, and read only after the loads that fill it have landed; the one
barrier per step (`s_waitcnt vmcnt(8) lgkmcnt(0); s_barrier`) is what orders
both.  A race would give wrong results only now and then, which the parity
tests cannot rule out, so this test proves the absence of one:

* a model of the ring, written from the kernel's source order (prologue,
  general and lean steps, K tail, the two steps that start the next tile,
  the epilogue's staging of C through two slots), emits each wave's LDS
  events: loads into a slot (with the content they carry), reads expecting
  a content, staging writes, and barriers with their vmcnt (the epilogue's
  global stores count in the same in-order counter, so leaving them out
  only makes the model wait for less than the kernel does);
* the checker splits the program into epochs at the barriers (every wave is
  in the same epoch between two barriers, anywhere within it) and requires
  that every read finds the expected content, landed in an earlier epoch,
  and that no write into a slot shares an epoch with reads of its old
  content or with a write still in flight;
* the same checker covers the one-tile hand-ordered kernels with an S-stage
  ring (the launch plan's 256 x 128 and 128 x 128 kernels), modelled the
  same way from their source order;
* the lean K loop of the built code object is read back and must issue
  exactly the model's schedule for its five steps: the load slots (from M0),
  the barrier after each step's first sub-step with vmcnt(8) lgkmcnt(0), and
  each fragment read's slot half and fragment index, with the same base
  register always standing for the same slot pair.
"""
from __future__ import annotations

import re

import pytest

import _isa
from dense_fp16_gemm_04_amd import binding

SLOTS = 5
LOADS = 8       # global->LDS loads per sub-step and wave (A_LOADS)
FRAGS = 8       # fragment reads per operand and sub-step (FM = FN)
SLOT_BYTES = 32768
FRAG_BYTES = 16 * 128  # 16 rows of 64 fp16 per fragment block
LEAN_SYMBOL = ("gemm_nt_f16_ordered_persist", "ILi256ELi256ELi64ELi2ELi2ELi2ELi1ELi0ELi16EEELi3ELi8ELi16EEE")


def ring_program(nk: int, tiles: int) -> list:
    """One wave's LDS events for `tiles` tiles of nk K steps each, in program
    order: ("load", slot, content), ("read", slot, content), ("write", slot,
    content), ("bar", vmcnt).  Contents: ("A"|"B", tile, step) or ("C", tile)."""
    ev = []
    adv = lambda s: (s + 2) % SLOTS  # noqa: E731

    def load(slot, what):
        ev.extend([("load", slot % SLOTS, what)] * LOADS)

    def read(slot, what):
        ev.extend([("read", slot % SLOTS, what)] * FRAGS)

    def step(sa, t, k, lt, ls, last):
        """Compute step k of tile t at ring position sa, loading step ls of
        tile lt (the loads of a step past K carry zeros, still loads)."""
        read(sa + 1, ("B", t, k))           # sub-step 0: set 1 of this step
        read(sa, ("A", t, k))
        load(sa + 4, ("A", lt, ls))
        ev.append(("bar", LOADS))           # all but the last 8 loads landed
        if not last:                        # sub-step 1: set 0 of the next step
            read(sa + 3, ("B", t, k + 1))
            read(sa + 2, ("A", t, k + 1))
            load(sa, ("B", lt, ls))

    # prologue: steps 0 and 1 of the first tile, wait for step 0
    load(0, ("A", 0, 0)); load(1, ("B", 0, 0)); load(2, ("A", 0, 1)); load(3, ("B", 0, 1))
    ev.append(("bar", 2 * LOADS))
    read(1, ("B", 0, 0)); read(0, ("A", 0, 0))
    sa = 0
    for t in range(tiles):
        for k in range(nk - 2):             # general and lean steps, K tail
            step(sa, t, k, t, k + 2, False)
            sa = adv(sa)
        step(sa, t, nk - 2, t + 1, 0, False)  # loads the next tile's step 0
        sa = adv(sa)
        step(sa, t, nk - 1, t + 1, 1, True)   # loads its step 1's A; no reads after
        for _ in range(2):                  # epilogue: C through slots sa, sa + 1
            ev.extend([("write", sa, ("C", t)), ("write", (sa + 1) % SLOTS, ("C", t))])
            ev.append(("bar", 63))
            ev.extend([("read", sa, ("C", t)), ("read", (sa + 1) % SLOTS, ("C", t))])
            ev.append(("bar", 63))
        if t == tiles - 1:
            break
        load(sa, ("B", t + 1, 1))
        sa = adv(sa)
        read(sa + 1, ("B", t + 1, 0)); read(sa, ("A", t + 1, 0))
    return ev


def races(ev) -> list:
    """Violations of the ordering rules in one wave's program (every wave
    runs the same program; the checks are per slot, over all waves)."""
    out = []
    epoch = 0
    issued = []          # load indices in issue order
    landed = {}          # load index -> epoch from which it is visible
    last_write = {}      # slot -> (event index, kind, content, epoch issued)
    readers = {}         # slot -> epochs of reads of the current content
    for i, e in enumerate(ev):
        kind = e[0]
        if kind == "bar":
            # every load but the last e[1] of each wave has landed; all LDS
            # reads and writes issued before it are done
            for j in issued[:max(0, len(issued) - e[1])]:
                landed.setdefault(j, epoch + 1)
            epoch += 1
            continue
        slot, what = e[1], e[2]
        if kind == "read":
            w = last_write.get(slot)
            if w is None or w[2] != what:
                out.append((i, "read of %s in slot %d finds %s" % (what, slot, None if w is None else w[2])))
                continue
            visible = landed.get(w[0]) if w[1] == "load" else w[3] + 1
            if visible is None or visible > epoch:
                out.append((i, "read of %s in slot %d before it has landed" % (what, slot)))
            readers.setdefault(slot, []).append(epoch)
        else:
            w = last_write.get(slot)
            if w is not None and w[2] != what:
                # a new content: its write window must not share an epoch
                # with reads of the old content or with the old write
                if any(r >= epoch for r in readers.get(slot, [])):
                    out.append((i, "write of %s into slot %d while %s is still read" % (what, slot, w[2])))
                old = landed.get(w[0]) if w[1] == "load" else w[3] + 1
                if old is None or old > epoch:
                    out.append((i, "write of %s into slot %d while %s may still land" % (what, slot, w[2])))
                readers[slot] = []
            if kind == "load":
                issued.append(i)
            # (pieces of one content land in issue order: the last one decides)
            last_write[slot] = (i, kind, what, epoch)
    return out


@pytest.mark.parametrize("nk", [2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 16, 127, 128, 129])
@pytest.mark.parametrize("tiles", [1, 2, 3, 4, 5])
def test_ring_has_no_races(nk, tiles):
    ev = ring_program(nk, tiles)
    assert races(ev) == []
    # every content that is computed is read: the model is not vacuous
    reads = {e[2] for e in ev if e[0] == "read"}
    for t in range(tiles):
        for k in range(nk):
            assert ("A", t, k) in reads and ("B", t, k) in reads


def stage_program(nk: int, stages: int, per_step: int = 4) -> list:
    """One loading wave's LDS events in the one-tile hand-ordered kernel with
    an S-stage ring (the 256 x 128 and 128 x 128 kernels of the launch plan):
    each stage holds the A and B tiles of one step, `per_step` loads per
    step and wave.  Every stage is filled first; step ks reads its second K
    half from its stage, waits for all but the last S - 2 steps' loads,
    reads the next step's first K half and loads step ks + S into the stage
    it has left (loads past the end of K bring zeros into stages the last
    steps still read into unused registers).  Then every load is waited for,
    all waves meet, and C is staged through the ring."""
    ev = []

    def load(stage, k):
        ev.extend([("load", stage, ("AB", k))] * per_step)

    def read(stage, k):
        ev.extend([("read", stage, ("AB", k))] * FRAGS)

    for st in range(stages):
        load(st, st)
    ev.append(("bar", per_step * (stages - 1)))
    read(0, 0)
    cur = 0
    for ks in range(nk):
        nxt = (cur + 1) % stages
        read(cur, ks)
        ev.append(("bar", per_step * (stages - 2)))
        read(nxt, ks + 1)
        load(cur, ks + stages)
        cur = nxt
    ev.append(("bar", 0))  # s_waitcnt vmcnt(0) and __syncthreads before the epilogue
    for st in range(stages):
        ev.append(("write", st, ("C",)))
    ev.append(("bar", 0))
    for st in range(stages):
        ev.append(("read", st, ("C",)))
    return ev


@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 6, 7, 16, 129])
def test_stage_ring_has_no_races(stages, nk):
    ev = stage_program(nk, stages)
    assert races(ev) == []
    if nk >= 2 and stages >= 3:
        # the steps' barriers (not the prologue's) with a window one load
        # wider let a read see a load still in flight
        first = next(i for i, e in enumerate(ev) if e[0] == "bar")
        weak = [("bar", e[1] + 1) if e[0] == "bar" and i > first and e[1] > 0 else e for i, e in enumerate(ev)]
        assert any("landed" in m for _, m in races(weak))


def test_checker_finds_planted_races():
    """Each rule fires on a program with one mistake planted."""
    ev = ring_program(6, 2)
    bars = [i for i, e in enumerate(ev) if e[0] == "bar" and e[1] == LOADS]
    # a step's barrier that waits for every load but the last 16 lets the
    # next step read data that may not have landed
    weak = list(ev)
    weak[bars[3]] = ("bar", 2 * LOADS)
    assert any("landed" in m for _, m in races(weak))
    # dropping a barrier lets a load overwrite a slot still being read
    dropped = ev[:bars[2]] + ev[bars[2] + 1:]
    assert any("still read" in m or "landed" in m for _, m in races(dropped))
    # loads of a second sub-step moved before the barrier overwrite the A
    # tile that the first sub-step is still reading
    group = [i for i, e in enumerate(ev) if e[0] == "load" and e[2] == ("B", 0, 2)]
    assert group[0] > bars[0]  # (so removing the group leaves the barrier's index as it was)
    rest = [e for i, e in enumerate(ev) if i not in group]
    early = rest[:bars[0]] + [ev[i] for i in group] + rest[bars[0]:]
    assert any("still read" in m for _, m in races(early))
    # a load into the wrong slot leaves a read with the wrong content
    wrong = [("load", (e[1] + 1) % SLOTS, e[2]) if e[0] == "load" and e[2] == ("A", 0, 2) else e for e in ev]
    assert any("finds" in m for _, m in races(wrong))


def _lean_loop_events(asm):
    """The lean loop's LDS events in issue order: ("read", base register,
    immediate), ("load", slot), ("bar", waitcnt text)."""
    lines = asm.splitlines()
    start = [i for i, l in enumerate(lines) if l.endswith(">:") and all(p in l for p in LEAN_SYMBOL)][0]
    ins = _isa.kernel(asm, LEAN_SYMBOL)
    bounds = None
    for a, _, t in ins:
        if t is not None and t <= a and sum(1 for x, m, _ in ins if t <= x <= a and m.startswith("v_mfma")) == 640:
            bounds = (t, a)
            break
    assert bounds, "no five-step loop in the lean kernel"
    ev, m0, prev = [], None, ""
    for l in lines[start + 1:]:
        if not l.strip():
            break
        m = re.match(r"\s+(\S+)(.*?)//\s*([0-9A-F]+):", l)
        if not m or not bounds[0] <= int(m.group(3), 16) <= bounds[1]:
            continue
        mn, ops = m.group(1), m.group(2).strip()
        if mn == "ds_read_b128":
            r = re.match(r"v\[\d+:\d+\],\s*(v\d+)(?:\s+offset:(\d+))?", ops)
            ev.append(("read", r.group(1), int(r.group(2) or 0)))
        elif mn in ("s_add_i32", "s_mov_b32") and ops.startswith("m0,"):
            imm = re.search(r",\s*(0x[0-9a-f]+|\d+)\s*$", ops) if mn == "s_add_i32" else None
            m0 = int(imm.group(1), 0) if imm else 0
        elif mn == "buffer_load_dwordx4":
            off = re.search(r"offset:(\d+)", ops)
            ev.append(("load", (m0 + int(off.group(1) if off else 0)) // SLOT_BYTES))
        elif mn == "s_barrier":
            ev.append(("bar", prev))
        if mn == "s_waitcnt":
            prev = ops
    return ev


def test_lean_loop_issues_the_model_schedule(tmp_path):
    ev = _lean_loop_events(_isa.disassemble(binding.library_path(), tmp_path))
    # the model's five steps from ring position 0, at fragment granularity
    want = []
    for s in (0, 2, 4, 1, 3):
        for sub, (ra, rb, kk, to) in enumerate([(s, s + 1, 1, s + 4), (s + 2, s + 3, 0, s)]):
            want += [("read", rb % SLOTS, "B", kk, i) for i in range(FRAGS)]
            want += [("read", ra % SLOTS, "A", kk, FRAGS - 1 - i) for i in range(FRAGS)]
            want += [("load", to % SLOTS)] * LOADS
            if sub == 0:
                want.append(("bar",))
    got_reads = [e for e in ev if e[0] == "read"]
    got_loads = [e[1] for e in ev if e[0] == "load"]
    assert [e[1] for e in want if e[0] == "load"] == got_loads
    # reads: slot half and fragment index from the immediate; the base
    # register stands for one (slot pair, operand, K half) throughout
    want_reads = [e for e in want if e[0] == "read"]
    assert len(got_reads) == len(want_reads)
    base_of = {}
    for (_, slot, op, kk, idx), (_, reg, imm) in zip(want_reads, got_reads):
        assert imm // SLOT_BYTES == slot % 2 and (imm % SLOT_BYTES) // FRAG_BYTES == idx, (slot, op, idx, imm)
        assert base_of.setdefault((slot // 2, op, kk), reg) == reg, (slot, op, kk, reg)
    assert len(set(base_of.values())) == len(base_of)
    # one barrier per step, after the first sub-step's 16 reads and 8 loads,
    # waiting for all but the last 8 loads and for every LDS access: between
    # barriers lie a second sub-step and the next step's first (reads and
    # loads interleave within a sub-step)
    bars = [i for i, e in enumerate(ev) if e[0] == "bar"]
    assert len(bars) == 5 and all(ev[b][1] == "vmcnt(8) lgkmcnt(0)" for b in bars), [ev[b] for b in bars]
    cuts = [-1] + bars + [len(ev)]
    segments = [ev[a + 1:b] for a, b in zip(cuts, cuts[1:])]
    per = [(sum(e[0] == "read" for e in seg), sum(e[0] == "load" for e in seg)) for seg in segments]
    assert per == [(2 * FRAGS, LOADS)] + [(4 * FRAGS, 2 * LOADS)] * 4 + [(2 * FRAGS, LOADS)], per
