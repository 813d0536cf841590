"""The LDS ring schedule of the bf16 attention kernel has no cross-wave race (CPU only).

The library exports the schedule the kernel itself follows (mla_debug_attn_schedule: for each
iteration, the ring buffer its direct-to-LDS loads write, and whether a workgroup barrier closes
it). This test lays the kernel's program out as phases (the stretches between workgroup barriers;
every wave runs the same sequence of barriers) and checks, for 1..40 tiles per key range:

* every read of a tile comes in a phase after the one in which each wave's loads of that tile were
  retired by a wait on the vector-memory counter (loads retire in issue order);
* every load into a buffer is issued in a phase strictly after every cross-wave read of what the
  buffer held before (a load may land any time between its issue and its retirement), and a
  load that carries no data (issued past the last tile) is retired before any later read of live
  data in its buffer;
* for every load, the barrier that orders it after the last reader of the previous contents is
  named (the barrier closing that reader's phase).

A schedule with the defect the kernel once had (the last iteration's dataless loads aimed at the
buffer of tile ntiles-2, with no barrier after that tile's weighted sum) must be reported racy.
"""
import pytest

from deepseek_mla_latent_amd import binding

lib = pytest.importorskip("deepseek_mla_latent_amd.binding").load_library()

NBUF = 4


def walk(ntiles, dma_buffer, barrier_after):
    """Events of one wave's program: ('load', buf, tile or None, phase), ('read', buf, tile, phase),
    ('retire', group, phase), with phases counted by the barriers passed."""
    phase = 0
    groups = []   # [buf, tile or None, issue phase, retire phase]
    retired = 0   # groups [0, retired) have been waited for
    reads = []    # (buf, tile, phase)
    barriers = []  # phase each barrier closes

    def issue(buf, tile):
        groups.append([buf, tile, phase, None])

    def wait(younger):
        nonlocal retired
        upto = max(len(groups) - younger, retired)
        for g in groups[retired:upto]:
            g[3] = phase
        retired = upto

    def barrier(name):
        nonlocal phase
        barriers.append((name, phase))
        phase += 1

    # prologue: the query rows pass through the tile area (wave-local), then the page ids
    barrier("query")
    for t in range(min(NBUF - 1, ntiles)):
        issue(t % NBUF, t)
    wait(min(ntiles - 1, 2))
    barrier("tile 0 landed")
    reads.append((0, 0, phase))                      # scores of tile 0
    if ntiles > 1:
        wait(1 if ntiles > 2 else 0)
        barrier("tile 1 landed")
    for t in range(ntiles):
        if t + 1 < ntiles:
            reads.append(((t + 1) % NBUF, t + 1, phase))  # scores of tile t+1 (past the end: unused)
        issue(dma_buffer[t], t + 3 if t + 3 < ntiles else None)
        reads.append((t % NBUF, t, phase))            # weighted sum of tile t
        if barrier_after[t]:
            wait(1)
            barrier(f"after iteration {t}")
    wait(0)
    barrier("epilogue")
    return groups, reads, barriers, phase


def check(ntiles, dma_buffer, barrier_after):
    """Returns a list of problems (empty when the schedule is race free) and the ordering barrier
    of each load."""
    groups, reads, barriers, end_phase = walk(ntiles, dma_buffer, barrier_after)
    problems, ordered_by = [], []
    landed = {g[1]: g[3] for g in groups if g[1] is not None}
    for buf, tile, ph in reads:
        if tile not in landed or landed[tile] is None or landed[tile] >= ph:
            problems.append(f"tile {tile} read in phase {ph} before its loads retired ({landed.get(tile)})")
    for gi, (buf, tile, issue_ph, retire_ph) in enumerate(groups):
        if retire_ph is None:
            problems.append(f"load group {gi} never retired")
            continue
        # the previous contents of buf: the latest tile loaded there before this group
        prev = [g for g in groups[:gi] if g[0] == buf and g[1] is not None]
        if prev:
            ptile = prev[-1][1]
            last_read = max((ph for b, t, ph in reads if t == ptile), default=-1)
            if last_read >= issue_ph:
                problems.append(f"load of {'tile ' + str(tile) if tile is not None else 'no data'} into buffer {buf} "
                                f"in phase {issue_ph} races with reads of tile {ptile} in phase {last_read}")
            else:
                ordered_by.append((gi, barriers[last_read][0]))
        else:
            ordered_by.append((gi, "query"))
        if tile is None:
            # no live read of this buffer may overlap the dataless load's flight
            for b, t, ph in reads:
                if b == buf and issue_ph <= ph <= retire_ph:
                    problems.append(f"dataless load into buffer {buf} (phases {issue_ph}-{retire_ph}) overlaps a "
                                    f"read of tile {t} in phase {ph}")
    assert end_phase == len(barriers)
    return problems, ordered_by


@pytest.mark.parametrize("ntiles", range(1, 41))
def test_ring_schedule_is_race_free(ntiles):
    bufs, bars = binding.mla_debug_attn_schedule(ntiles)
    assert len(bufs) == ntiles and all(0 <= b < NBUF for b in bufs)
    for t in range(ntiles):  # live loads go where the ring puts their tile
        if t + 3 < ntiles:
            assert bufs[t] == (t + 3) % NBUF
    problems, ordered_by = check(ntiles, bufs, bars)
    assert not problems, problems
    assert len(ordered_by) == min(3, ntiles) + ntiles  # every load has an ordering barrier


def test_the_old_schedule_is_reported_racy():
    """The defect: every iteration aimed its loads at (t + 3) % 4, the last one included."""
    for ntiles in range(2, 41):
        bufs = [(t + 3) % NBUF for t in range(ntiles)]
        bars = [t + 2 < ntiles for t in range(ntiles)]
        problems, _ = check(ntiles, bufs, bars)
        assert any("races with reads of tile" in p for p in problems), ntiles
    # one tile: the lone dataless load goes to a buffer nobody uses, which is fine either way
    assert not check(1, [3], [False])[0]


def test_schedule_argument_errors():
    import ctypes
    a = (ctypes.c_int32 * 1)()
    assert lib.mla_debug_attn_schedule(0, a, a) == -2
    assert lib.mla_debug_attn_schedule(1, None, a) == -1
