"""The LDS ring schedule of the bf16 attention kernel has no cross-wave race (CPU only).

The library exports the buffers the kernel itself uses (mla_debug_attn_schedule: for each
iteration u, the ring-A and ring-B buffers its loads write, which hold tile u + 2, and the ring-P
buffer the probabilities of tile u go to). This test lays the kernel's program out as phases (the
stretches between workgroup barriers; every wave passes the same barriers in the same order) and
checks, for 1..40 tiles per key range:

* every read of a tile comes in a phase after the one in which each wave's loads of that tile were
  retired by a wait on the vector-memory counter (loads retire in issue order);
* every load into a buffer is issued in a phase strictly after every cross-wave read of what the
  buffer held before (a load may land at any time between its issue and its retirement), and a
  load that carries no data (issued past the last tile) overlaps no read of its buffer at all;
* every write of probabilities comes in a phase after the last read of what its buffer held, and
  every read of them in a phase after the write;
* for every write, the barrier that orders it after the last reader of the previous contents is
  named.

Each ring one buffer shallower than the kernel's (A 3, B 2, P 1) must be reported racy.

The phases, as the kernel runs them:
  query      the query rows pass through ring A (each wave reads only its own), page ids to LDS
  tile 0     loads of tiles 0 and 1 issued; each wave waits for its tile-0 loads
  iter u     scores of tile u (A, B); loads of tile u + 2; weighted sum of tile u - 1 (A, P);
             probabilities of tile u written (P); wait for the loads of tile u + 1; barrier Z(u)
  last sum   weighted sum of tile ntiles - 1 (A, P); wait for every load; barrier
  epilogue   the output rows are staged through the ring area
"""
import pytest

from deepseek_mla_latent_amd import binding

lib = pytest.importorskip("deepseek_mla_latent_amd.binding").load_library()

NA, NB, NP, AHEAD = 4, 3, 2, 2


def kernel_schedule(ntiles):
    a, b, p = binding.mla_debug_attn_schedule(ntiles)
    return a, b, p


def walk(ntiles, a_of_iter, b_of_iter, p_of_iter, a_of_tile, b_of_tile):
    """Events of one wave's program with phase numbers; a_of_tile / b_of_tile place tiles 0 and 1
    (loaded by the prologue), the per-iteration arrays place everything the loop touches."""
    phase = 0
    groups = []     # dicts: ring buffers, tile (None = no data), issue / retire phase
    retired = 0
    reads = []      # (ring, buf, content, phase); content = ("tile", j) or ("p", j)
    writes_p = []   # (buf, j, phase)
    barriers = []   # names, index = the phase each one closes

    def issue(tile, abuf, bbuf):
        groups.append(dict(tile=tile if tile < ntiles else None, A=abuf, B=bbuf, issue=phase, retire=None))

    def wait(younger):
        nonlocal retired
        upto = max(len(groups) - younger, retired)
        for g in groups[retired:upto]:
            g["retire"] = phase
        retired = upto

    def barrier(name):
        nonlocal phase
        barriers.append(name)
        phase += 1

    barrier("query")
    issue(0, a_of_tile(0), b_of_tile(0))
    issue(1, a_of_tile(1), b_of_tile(1))
    wait(1)
    barrier("tile 0")
    for u in range(ntiles):
        reads.append(("A", a_of_tile(u), ("tile", u), phase))
        reads.append(("B", b_of_tile(u), ("tile", u), phase))
        issue(u + AHEAD, a_of_iter[u], b_of_iter[u])
        if u >= 1:
            reads.append(("A", a_of_tile(u - 1), ("tile", u - 1), phase))
            reads.append(("P", p_of_iter[u - 1], ("p", u - 1), phase))
        writes_p.append((p_of_iter[u], u, phase))
        wait(1)
        barrier(f"Z({u})")
    reads.append(("A", a_of_tile(ntiles - 1), ("tile", ntiles - 1), phase))
    reads.append(("P", p_of_iter[ntiles - 1], ("p", ntiles - 1), phase))
    wait(0)
    barrier("last sum")
    return groups, reads, writes_p, barriers, phase


def check(ntiles, a_of_iter, b_of_iter, p_of_iter, a_of_tile, b_of_tile):
    groups, reads, writes_p, barriers, end = walk(ntiles, a_of_iter, b_of_iter, p_of_iter, a_of_tile, b_of_tile)
    problems, ordered_by = [], []
    retire_of = {g["tile"]: g["retire"] for g in groups if g["tile"] is not None}
    for ring, buf, (kind, j), ph in reads:
        if kind == "tile" and not (retire_of.get(j) is not None and retire_of[j] < ph):
            problems.append(f"tile {j} read from ring {ring} in phase {ph}, its loads retired in {retire_of.get(j)}")
    for gi, g in enumerate(groups):
        if g["retire"] is None:
            problems.append(f"load group {gi} never retired")
            continue
        for ring in ("A", "B"):
            buf = g[ring]
            prev = [h for h in groups[:gi] if h[ring] == buf and h["tile"] is not None]
            if prev:
                pt = prev[-1]["tile"]
                last = max((ph for r, bb, c, ph in reads if r == ring and c == ("tile", pt)), default=-1)
                if last >= g["issue"]:
                    problems.append(f"loads of {'tile %d' % g['tile'] if g['tile'] is not None else 'no data'} into "
                                    f"ring {ring} buffer {buf} (phase {g['issue']}) race with reads of tile {pt} "
                                    f"(phase {last})")
                else:
                    ordered_by.append((ring, gi, barriers[last]))
            else:
                ordered_by.append((ring, gi, "query"))
            if g["tile"] is None:
                for r, bb, c, ph in reads:
                    if r == ring and bb == buf and g["issue"] <= ph <= g["retire"]:
                        problems.append(f"dataless loads into ring {ring} buffer {buf} (phases {g['issue']}-"
                                        f"{g['retire']}) overlap a read of {c} in phase {ph}")
    for buf, j, ph in writes_p:
        earlier = [jj for bb, jj, pp in writes_p if bb == buf and jj < j]
        if earlier:
            last = max(pp for r, bb, c, pp in reads if r == "P" and c == ("p", earlier[-1]))
            if last >= ph:
                problems.append(f"probabilities of tile {j} written to P buffer {buf} in phase {ph} race with "
                                f"reads of tile {earlier[-1]}'s (phase {last})")
            else:
                ordered_by.append(("P", j, barriers[last]))
        rd = [pp for r, bb, c, pp in reads if r == "P" and c == ("p", j)]
        if not rd or min(rd) <= ph:
            problems.append(f"probabilities of tile {j} read in the phase they are written")
    assert end == len(barriers)
    return problems, ordered_by


@pytest.mark.parametrize("ntiles", range(1, 41))
def test_ring_schedule_is_race_free(ntiles):
    a, b, p = kernel_schedule(ntiles)
    assert len(a) == len(b) == len(p) == ntiles
    assert all(0 <= v < NA for v in a) and all(0 <= v < NB for v in b) and all(0 <= v < NP for v in p)
    problems, ordered_by = check(ntiles, a, b, p, lambda j: j % NA, lambda j: j % NB)
    assert not problems, problems
    # iteration u loads into the buffers of tile u + 2, the same function the kernel places tiles with
    assert a == [(u + AHEAD) % NA for u in range(ntiles)] and b == [(u + AHEAD) % NB for u in range(ntiles)]
    assert len(ordered_by) == 2 * (ntiles + 2) + ntiles - min(ntiles, NP)


@pytest.mark.parametrize("ring", ["A", "B", "P"])
def test_a_shallower_ring_is_reported_racy(ring):
    na, nb, np_ = NA - (ring == "A"), NB - (ring == "B"), NP - (ring == "P")
    for ntiles in range(4, 41):
        a = [(u + AHEAD) % na for u in range(ntiles)]
        b = [(u + AHEAD) % nb for u in range(ntiles)]
        p = [u % np_ for u in range(ntiles)]
        problems, _ = check(ntiles, a, b, p, lambda j: j % na, lambda j: j % nb)
        assert problems, (ring, ntiles)


def test_schedule_argument_errors():
    import ctypes
    x = (ctypes.c_int32 * 1)()
    assert lib.mla_debug_attn_schedule(0, x, x, x) == -2
    assert lib.mla_debug_attn_schedule(1, None, x, x) == -1
