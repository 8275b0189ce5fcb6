"""A host-side model of the forward kernel's LDS rings (CPU only).

The fused forward streams K and V tiles through rings of RING LDS buffers
per tensor: iteration t starts the direct-to-LDS copies of K(t + KLEAD) and
V(t + VLEAD), forms S of tile t + 1 from K buffer (t + 1) % RING and P.V of
tile t - 1 from V buffer (t - 1) % RING; each of the workgroup's waves copies
its share of every tile, and barriers (with waits for the wave's own
copies) order the copies against the other waves' reads.

The model replays that schedule for every wave as a list of events --
copy issued, wait for all but the n youngest copies, barrier, read -- and
checks two things:
  * every read sees its tile complete: each wave's share of the copy was
    waited for before a barrier the reading wave passed before the read;
  * no copy overwrites a buffer while any wave may still read the tile it
    held: every read of the old tile lies in an earlier barrier epoch than
    the copy that replaces it.
Waves that skip an iteration's products (past the causal diagonal or past
the end of the queries) skip its reads but keep its copies and barriers;
the model covers every subset of skipped iterations per wave that the
kernel's rule allows (a wave skips from some iteration on).  A causal
workgroup processes two query blocks in turn, separated by a barrier.

The schedule's constants (lead distances, where the barriers are) are read
from the kernel source, so the model checks the schedule the kernel runs.
A schedule without the barrier after iteration 0 (a copy at iteration 1
refilling K buffer 0 while a slower wave still reads K(0) from the
prologue) is shown to fail.
"""
import itertools
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "exact_io_aware_40_amd", "csrc", "attn_fwd_kernel.h")


def kernel_schedule():
    """The ring's parameters as the kernel source states them."""
    text = open(SRC).read()
    occ = int(re.search(r"constexpr int OCC = (\d+);", text).group(1))
    m = re.search(r"constexpr int RING = \(160 \* 1024 / OCC\) / \(2 \* 8192\);", text)
    assert m, "the ring size formula changed; update the model"
    ring = (160 * 1024 // occ) // (2 * 8192)
    klead = ring - int(re.search(r"constexpr int KLEAD = RING - (\d+);", text).group(1))
    vlead = ring - int(re.search(r"constexpr int VLEAD = RING - (\d+);", text).group(1))
    pairb = "constexpr bool PAIRB = RING >= 5;" in text
    t0_barrier = re.search(r"else if \(t == 0\) \{[^}]*barrier_only\(\);", text, flags=re.S) is not None
    # after the loop: the wave's own copies waited for, then a barrier, before
    # the epilogue stages O through the rings' LDS
    epi = re.search(r"\n        wait_vmem\(\);\n        __syncthreads\(\);\n", text) is not None
    return dict(ring=ring, klead=klead, vlead=vlead, pairb=pairb, t0_barrier=t0_barrier, epi_barrier=epi)


def wave_events(ring, klead, vlead, pairb, t0_barrier, ntiles, skip_from, items=1, epi_barrier=True):
    """The event list of one wave.  Events: ("copy", tensor, tile, buffer),
    ("wait", n) -- all but the n youngest copies complete --, ("barrier",),
    ("read", tensor, tile, buffer).  skip_from: first iteration whose
    products the wave skips (ntiles + 1: none).  Mirrors the kernel: the
    prologue issues K(0), K(1), then the copies iterations -vlead .. -1
    would start; clears V buffer ring - 1 (tile -1, P = 0) by plain stores;
    waits for all but the youngest iteration's copies; barrier; reads K(0)
    for S of tile 0.  Iteration t = 0 .. ntiles: copies K(t + klead) and
    V(t + vlead) (only tiles < ntiles exist; a copy past the end is a
    zero-length copy that still counts), reads K(t + 1) and V(t - 1) unless
    skipped, then the barrier rule.  After the loop: wait for everything,
    the epilogue barrier (when the kernel has it), ("stage",) -- the wave
    writes its O tile over the rings' LDS and reads it back --, and between
    items a barrier."""
    ev = []
    per_iter_wait = 2 if pairb else 2 * (klead - 2)   # copies younger than those waited for
    for item in range(items):
        # a tile is named (item, index), so that the two items' tiles differ
        def copy(tensor, tile):
            ev.append(("copy", tensor, (item, tile), tile % ring))

        def read(tensor, tile):
            ev.append(("read", tensor, (item, tile), tile % ring))

        copy("K", 0)
        copy("K", 1)
        for t in range(-vlead, 0):
            copy("K", t + klead)
            copy("V", t + vlead)
        ev.append(("store", "V", (item, -1), ring - 1))
        ev.append(("wait", per_iter_wait))
        ev.append(("barrier",))
        read("K", 0)
        for t in range(ntiles + 1):
            copy("K", t + klead)
            copy("V", t + vlead)
            if t < skip_from:
                read("K", t + 1)
                read("V", t - 1)
            if not pairb or t % 2 == 1:
                ev.append(("wait", per_iter_wait))
                ev.append(("barrier",))
            elif t == 0 and t0_barrier:
                ev.append(("barrier",))
        ev.append(("wait", 0))
        if epi_barrier:
            ev.append(("barrier",))
        ev.append(("stage", item))
        if item + 1 < items:
            ev.append(("barrier",))
    return ev


def check(waves):
    """Raise AssertionError on a read of an incomplete tile or an overwrite
    of a tile some wave may still read.  waves: one event list per wave."""
    nb = [sum(1 for e in w if e[0] == "barrier") for w in waves]
    assert len(set(nb)) == 1, f"waves pass different numbers of barriers: {nb}"
    # per wave: epoch (barriers passed) of each event, and for every copy the
    # epoch of the wait that completed it (the wave's copies complete in order)
    info = []
    for w in waves:
        epoch, copies, done_at, evs = 0, [], {}, []
        for e in w:
            if e[0] == "barrier":
                epoch += 1
            elif e[0] == "copy":
                copies.append(len(evs))
            elif e[0] == "wait":
                keep = e[1]
                for ci in copies[:max(0, len(copies) - keep)]:
                    done_at.setdefault(ci, epoch)
            evs.append((e, epoch))
        for ci in copies:
            done_at.setdefault(ci, None)
        info.append((evs, done_at))
    # the k-th write into a buffer by each wave is the same generation:
    # (tensor, buffer) -> generation -> [tile, issue epoch per wave, epoch in
    # which each wave's share was complete]
    n = len(waves)
    gens = {}
    for wi, (evs, done_at) in enumerate(info):
        cnt = {}
        for idx, (e, ep) in enumerate(evs):
            if e[0] in ("copy", "store"):
                key = (e[1], e[3])
                g = cnt.get(key, 0)
                cnt[key] = g + 1
                gens.setdefault(key, {}).setdefault(g, [e[2], [None] * n, [None] * n])
                rec = gens[key][g]
                assert rec[0] == e[2], f"waves disagree on the tile of {key} generation {g}"
                rec[1][wi] = ep
                # a plain store completes at once (program order); a copy when waited
                rec[2][wi] = ep if e[0] == "store" else done_at[idx]
    # staging: every copy of the item (zero-length ones included) complete in
    # every wave before any wave stages O over the rings, and the next item's
    # copies start after every wave has staged
    for wi, (evs, done_at) in enumerate(info):
        for idx, (e, ep) in enumerate(evs):
            if e[0] != "stage":
                continue
            item = e[1]
            for wj, (evj, dj) in enumerate(info):
                for jdx, (e2, ep2) in enumerate(evj):
                    if e2[0] == "copy" and e2[2][0] == item:
                        d = dj[jdx]
                        assert d is not None and d < ep, (
                            f"wave {wi} stages O in epoch {ep} while wave {wj}'s copy of {e2[1]}{e2[2]} "
                            f"may still be writing LDS (complete in epoch {d})")
                    if e2[0] in ("copy", "store") and e2[2][0] > item:
                        assert ep2 > ep, (f"wave {wj} starts {e2[1]}{e2[2]} in epoch {ep2} while wave {wi} "
                                          f"stages O of item {item} (epoch {ep})")
    # reads: find the generation a read sees and check it
    for wi, (evs, _) in enumerate(info):
        for e, ep in evs:
            if e[0] != "read":
                continue
            key = (e[1], e[3])
            glist = gens.get(key, {})
            # the generation holding the tile read
            g = next((g for g, rec in glist.items() if rec[0] == e[2]), None)
            assert g is not None, f"wave {wi} reads {e[1]}({e[2]}) from buffer {e[3]}, never copied there"
            rec = glist[g]
            for wj in range(n):
                d = rec[2][wj]
                assert d is not None and (d < ep), (
                    f"wave {wi} reads {e[1]}({e[2]}) in epoch {ep} before wave {wj}'s share of it is "
                    f"complete and past a barrier (completed in epoch {d})")
            # the epilogue's staging of O overwrites the rings: every wave's
            # staging of this item must come after the read
            for wj, (evj, _) in enumerate(info):
                for e2, ep2 in evj:
                    if e2[0] == "stage" and e2[1] == e[2][0]:
                        assert ep2 > ep, (f"wave {wj} stages O over the rings in epoch {ep2} while wave "
                                          f"{wi} may still read {e[1]}({e[2]}) (epoch {ep})")
            nxt = glist.get(g + 1)
            if nxt is not None:
                for wj in range(n):
                    assert nxt[1][wj] is not None and nxt[1][wj] > ep, (
                        f"wave {wj} starts copying {e[1]}({nxt[0]}) into buffer {e[3]} in epoch "
                        f"{nxt[1][wj]} while wave {wi} may still read {e[1]}({e[2]}) there (epoch {ep})")


def run(sched, ntiles, skips, items=1):
    waves = [wave_events(sched["ring"], sched["klead"], sched["vlead"], sched["pairb"],
                         sched["t0_barrier"], ntiles, s, items, sched.get("epi_barrier", True)) for s in skips]
    check(waves)


def skip_patterns(ntiles, nwaves=4):
    """Every assignment of a first skipped iteration per wave among a few
    representative values (none, the last, the middle, 1, 0)."""
    cand = sorted({ntiles + 1, ntiles, max(1, ntiles // 2), 1, 0})
    return itertools.product(cand, repeat=nwaves)


def test_kernel_schedule_is_read():
    s = kernel_schedule()
    assert s["ring"] in (4, 5)
    assert s["klead"] == s["ring"] - 1
    assert s["epi_barrier"]


def test_epilogue_without_its_barrier_is_a_race():
    """Staging O over the rings right after the wave's own loop: another wave
    may still read its last tiles, or its last copies may still land."""
    s = dict(kernel_schedule(), epi_barrier=False)
    with pytest.raises(AssertionError, match="stages O"):
        run(s, 6, (7, 7, 7, 7))


@pytest.mark.parametrize("ntiles", [1, 2, 3, 4, 5, 6, 9, 12])
@pytest.mark.parametrize("items", [1, 2])
def test_kernel_ring_has_no_race(ntiles, items):
    s = kernel_schedule()
    for skips in skip_patterns(ntiles):
        run(s, ntiles, skips, items)


@pytest.mark.parametrize("ntiles", [2, 5, 8])
def test_four_buffer_ring_has_no_race(ntiles):
    """The four-buffer form: copies three (K) and one (V) iteration ahead, a
    wait and a barrier after every iteration."""
    s = dict(ring=4, klead=3, vlead=1, pairb=False, t0_barrier=False)
    for skips in skip_patterns(ntiles):
        run(s, ntiles, skips)


def test_missing_first_barrier_is_a_race():
    """The five-buffer ring without the barrier after iteration 0: iteration 1
    refills K buffer 0 in the same epoch in which a slower wave reads K(0)."""
    s = dict(kernel_schedule(), t0_barrier=False)
    assert s["ring"] == 5
    with pytest.raises(AssertionError, match="while wave"):
        run(s, 6, (7, 7, 7, 7))


def test_missing_wait_is_a_race():
    """Barriers without the waits for the waves' own copies: a tile is read
    before every wave's share of it has landed."""
    s = kernel_schedule()
    waves = [[e for e in wave_events(s["ring"], s["klead"], s["vlead"], s["pairb"], s["t0_barrier"], 6, 7)
              if e[0] != "wait" or e[1] == 0] for _ in range(4)]
    with pytest.raises(AssertionError, match="complete"):
        check(waves)


def test_too_short_lead_is_a_race():
    """K copied five iterations ahead into a ring of five: it would overwrite
    the buffer of the tile being read in the same iteration."""
    s = dict(kernel_schedule(), klead=5)
    with pytest.raises(AssertionError):
        run(s, 6, (7, 7, 7, 7))
