"""CPU checks of the single launch's work and copy tables
(dist_gemm_fused_tables, host only): their bookkeeping, and an event-driven
model of the persistent kernel's protocol run on them.

The model follows the kernel's rules: workgroup b takes items from queue
b mod nq in order; a tile of a quota segment claims its quota of list-0
pieces and copies them before its GEMM; a tile whose strip is incomplete
claims and copies list-0 pieces (then, for a strip of list 1, list-1
pieces) one at a time while it waits, and otherwise blocks until the strip
completes; a tile that starts its GEMM claims one list-1 piece, which
completes when the tile does (in-loop form); a workgroup with no items left
sweeps both lists.  It checks that no run of the protocol stalls (every
blocked workgroup is woken by a piece some running workgroup finishes),
that every tile of the grid runs exactly once and only after its strip is
complete, and that every piece is claimed exactly once and every staged
strip's counter reaches its target.  Times are model units: a tile 100, a
piece copied through LDS 2 per 128 KiB.
"""
import heapq
import itertools

import pytest

import communication_tensor_gemm_amd as dg

GROUP = 4  # tile rows (or columns) walked together in a segment's tile order


def order_tile(t, tiles_m, tiles_n):
    per_group = GROUP * tiles_n
    g = t // per_group
    first_m = g * GROUP
    gm = min(GROUP, tiles_m - first_m)
    w = t - g * per_group
    return first_m + w % gm, w // gm


def piece_step(tb, p):
    for h in tb["claim_steps"]:
        base, n = tb["steps"][h][6], tb["steps"][h][4]
        if base <= p < base + n:
            return h
    raise AssertionError(f"piece {p} outside every step")


def chunk_at(tb, h, c):
    _, strip0, nst, P, n_chunks, _, _ = tb["steps"][h]
    per_strip = tb["LG"] * P
    sp, rem = divmod(c, per_strip)
    return strip0 + sp, rem // P


def lists(tb, copy_local):
    n0, n1, nz = tb["n_list0"], tb["n_list1"], (tb["n_local"] if copy_local else 0)
    if n1 > 0:
        return [[0, n0], [n0, n0 + n1 + nz]]
    return [[0, n0 + nz], [n0 + nz, n0 + nz]]


def half_tail_tiles(n, slots):
    """Tiles of a last partial round that run as two half-height items."""
    rem = n % slots
    return rem if 0 < rem and 2 * rem <= slots else 0


def simulate(tb, L, nq, n_wg, copy_local=False, half_tail=True):
    """Run the protocol; return (tiles seen as (l, strip, other, half or -1),
    per-strip counters, claims, end time)."""
    S = len(tb["steps"])
    LG = tb["LG"]
    ranges = lists(tb, copy_local)
    claim = [r[0] for r in ranges]
    claimed = {}
    ctr = {}
    qctr = [0] * nq
    waiting = {}  # (lg, strip) -> [wg]
    done_tiles = []
    events = []
    seq = itertools.count()

    def complete(p):
        h = piece_step(tb, p)
        pos, lg = chunk_at(tb, h, p - tb["steps"][h][6])
        key = (lg, tb["strip_list"][pos])
        ctr[key] = ctr.get(key, 0) + 1
        if ctr[key] == tb["steps"][h][3]:
            for wg in waiting.pop(key, []):
                heapq.heappush(events, (now[0], next(seq), wg))

    def take(li, n):
        lo = claim[li]
        claim[li] = min(ranges[li][1], lo + n)
        for p in range(lo, claim[li]):
            assert p not in claimed, f"piece {p} claimed twice"
            claimed[p] = True
        return list(range(lo, claim[li]))

    def piece_time(p):
        h = piece_step(tb, p)
        nbytes = tb["steps"][h][0] * (1 if not tb["strided"] else 256 * tb["row_bytes"])
        return max(1, 2 * nbytes // (128 << 10))

    def workgroup(b):
        q = b % nq
        seg = tb["seg"][q]
        n_tiles = seg[-1]
        split = half_tail_tiles(n_tiles, n_wg // nq) if half_tail else 0
        whole, n_items = n_tiles - split, n_tiles + split
        while True:
            item = qctr[q]
            qctr[q] += 1
            if item >= n_items:
                break
            k = item if item < whole else whole + (item - whole) // 2
            hrow = -1 if item < whole else (item - whole) % 2
            g = max(i for i in range(len(seg) - 1) if seg[i] <= k)
            nst = tb["segs"][g][1]
            T2 = tb["segs"][g][2]
            qq, r = divmod(T2, nq)
            share, first = qq + (1 if q < r else 0), q * qq + min(q, r)
            i = k - seg[g]
            l, j = divmod(i, share)
            if tb["cols"]:
                ob, sp = order_tile(first + j, T2 // nst, nst)
            else:
                sp, ob = order_tile(first + j, nst, T2 // nst)
            pos = tb["segs"][g][0] + sp
            strip, h_own = tb["strip_list"][pos], tb["strip_step"][pos]
            own = tb["steps"][h_own]
            lg = 0 if LG == 1 else l
            quota = tb["segs"][g][3]
            if quota > 0:
                ps = take(0, quota)
                if ps:
                    yield ("delay", sum(piece_time(p) for p in ps))
                    for p in ps:
                        complete(p)
            if own[5]:
                key = (lg, strip)
                while ctr.get(key, 0) < own[3]:
                    ps = take(0, 1)
                    if not ps and own[6] >= ranges[1][0]:
                        ps = take(1, 1)
                    if ps:
                        yield ("delay", piece_time(ps[0]))
                        complete(ps[0])
                    else:
                        waiting.setdefault(key, []).append(b)
                        yield ("block", None)
                assert ctr.get(key, 0) >= own[3]
            mine = take(1, 1) if tb["loop"] else []
            done_tiles.append((l, strip, ob, hrow))
            yield ("delay", 100 if hrow < 0 else 50)
            for p in mine:
                complete(p)
        for li in (0, 1):
            while claim[li] < ranges[li][1]:
                ps = take(li, 4)
                yield ("delay", sum(piece_time(p) for p in ps))
                for p in ps:
                    complete(p)

    now = [0]
    gens = {b: workgroup(b) for b in range(n_wg)}
    for b in range(n_wg):
        heapq.heappush(events, (0, next(seq), b))
    finished = set()
    while events:
        t, _, b = heapq.heappop(events)
        now[0] = t
        try:
            kind, arg = next(gens[b])
        except StopIteration:
            finished.add(b)
            continue
        if kind == "delay":
            heapq.heappush(events, (t + arg, next(seq), b))
    stalled = [b for b in range(n_wg) if b not in finished]
    assert not stalled, f"{len(stalled)} workgroups never finish (waiting on {list(waiting)[:4]})"
    return done_tiles, ctr, claimed, now[0]


def check_tables(tb, M, N, L, TP, nq, n_wg, copy_ahead):
    S = TP
    steps = tb["steps"]
    # claim order: steps 1 .. S-1, then 0, with contiguous piece ranges
    assert tb["claim_steps"] == list(range(1, S)) + [0]
    base = 0
    for h in tb["claim_steps"]:
        piece, strip0, nst, P, n_chunks, wait, b = steps[h]
        assert b == base and n_chunks == nst * tb["LG"] * P
        assert wait == (1 if h else 0)
        if tb["strided"]:
            assert P * piece >= tb["height"] > (P - 1) * piece
        else:
            assert piece % 16 == 0 and P * piece >= tb["strip_bytes"] > (P - 1) * piece
        base += n_chunks
    assert base == tb["n_list0"] + tb["n_list1"] + tb["n_local"]
    assert tb["n_local"] == steps[0][4]
    # the strip list is step by step and covers every strip once
    assert sorted(tb["strip_list"]) == list(range(tb["n_strips"]))
    for h in range(S):
        _, strip0, nst = steps[h][:3]
        assert all(tb["strip_step"][p] == h for p in range(strip0, strip0 + nst))
    # list 0: the staged steps the first round reads
    per_q = n_wg // nq
    reached = set()
    for q in range(nq):
        seg = tb["seg"][q]
        for g in range(tb["n_segs"]):
            if seg[g + 1] > seg[g] and seg[g] < per_q:
                reached.add(g)
    seg_last_step = {}
    for h in range(S):
        for g, (strip0, nst, _, _) in enumerate(tb["segs"]):
            if nst and strip0 <= steps[h][1] < strip0 + nst:
                seg_last_step[g] = max(seg_last_step.get(g, 0), h)
    h1 = max(seg_last_step.get(g, 0) for g in reached)
    n0 = sum(steps[h][4] for h in range(1, S) if h <= h1 or not tb["loop"])
    assert tb["n_list0"] == n0
    if tb["loop"]:
        assert tb["n_list1"] > 0
        for h in range(h1 + 1, S):
            assert steps[h][0] <= tb["loop_capacity"]
    else:
        assert tb["n_list1"] == 0
    # quotas: the first copy_ahead segments, only when list 0 has pieces
    for g, (_, _, tiles, quota) in enumerate(tb["segs"]):
        if g < copy_ahead and tb["n_list0"] > 0:
            assert quota > 0
        else:
            assert quota == 0
    # queues: every segment's tiles (times L) split over the queues
    for g, (_, nst, tiles, _) in enumerate(tb["segs"]):
        assert sum(tb["seg"][q][g + 1] - tb["seg"][q][g] for q in range(nq)) == tiles * L


CASES = [
    # M, N, K, L, TP, schedule, dtype, shared_a, queues, step_group, copy_ahead, copy_chunk, n_wg
    (16384, 13312, 16384, 1, 8, "AG_ROT_A", "BF16_F32", 0, 8, 2, 1, 2 << 20, 256),   # bf16 AG-A TP=8
    (8192, 13312, 16384, 1, 8, "AG_ROT_B", "E4M3_BF16", 0, 8, 2, 1, 2 << 20, 256),   # e4m3 AG-B TP=8
    (8192, 8192, 3584, 1, 8, "RS_TILE_A_ROT_C", "BF16_F32", 0, 8, 2, 1, 2 << 20, 256),
    (16384, 8192, 8192, 1, 8, "AG_ROT_A", "F32", 0, 8, 2, 1, 2 << 20, 256),
    (8192, 8192, 3584, 1, 8, "RS_TILE_A_ROT_C", "BF16_F32", 0, 8, 1, 0, 2 << 20, 256),
    (8192, 8192, 3584, 1, 8, "RS_TILE_A_ROT_C", "BF16_F32", 0, 1, 7, 64, 4096, 256),
    (8192, 4096, 1024, 2, 8, "AG_ROT_A", "BF16_BF16", 1, 8, 2, 1, 2 << 20, 256),      # shared A, L = 2
    (4096, 8192, 1024, 1, 8, "AG_ROT_B", "BF16_BF16", 0, 8, 3, 2, 2 << 20, 64),
    (2048, 8192, 512, 1, 8, "RS_TILE_B_ROT_C", "F32", 0, 8, 2, 1, 65536, 256),        # column strips
    (512, 2048, 128, 3, 4, "RS_TILE_B_ROT_C", "BF16_F32", 0, 1, 1, 1, 4096, 16),
    (600, 520, 272, 1, 4, "AG_ROT_A", "BF16_BF16", 0, 8, 2, 1, 2 << 20, 256),         # no local strip
    (1024, 3328, 512, 1, 8, "AG_ROT_B", "E4M3_BF16", 0, 8, 2, 1, 2 << 20, 8),         # straddling strips
    (8192, 2048, 4096, 1, 16, "AG_ROT_A", "BF16_F32", 0, 8, 2, 1, 2 << 20, 64),
    (4096, 4096, 2048, 2, 8, "RS_TILE_A_ROT_C", "E4M3_F32", 0, 8, 2, 1, 2 << 20, 128),
]


@pytest.mark.parametrize("half_tail", [True, False])
@pytest.mark.parametrize("copy_local", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[5]}_{c[0]}x{c[1]}x{c[2]}_L{c[3]}_tp{c[4]}_q{c[8]}g{c[9]}a{c[10]}w{c[12]}"
                                            for c in CASES])
def test_tables_and_protocol(case, copy_local, half_tail):
    M, N, K, L, TP, sched, dtype, shared_a, nq, group, ahead, chunk, n_wg = case
    if copy_local and not sched.startswith("AG"):
        pytest.skip("the gathered image is returned for the all-gather schedules only")
    tb = dg.dist_gemm_fused_tables(M, N, K, L, TP, sched, dtype, shared_a, nq, group, ahead, chunk, n_wg)
    check_tables(tb, M, N, L, TP, nq, n_wg, ahead)
    tiles, ctr, claimed, t_end = simulate(tb, L, nq, n_wg, copy_local, half_tail)
    # every tile of the grid once, whole or as its two halves
    n_other = ((N if not tb["cols"] else M) + 255) // 256
    expect = sorted((l, s, o) for l in range(L) for s in range(tb["n_strips"]) for o in range(n_other))
    whole = [t[:3] for t in tiles if t[3] < 0]
    halves = sorted(t for t in tiles if t[3] >= 0)
    assert halves[0::2] == sorted(t[:3] + (0,) for t in halves[1::2]) or not halves
    assert [t[3] for t in halves] == [0, 1] * (len(halves) // 2)
    assert sorted(whole + [t[:3] for t in halves[0::2]]) == expect
    if not half_tail:
        assert not halves
    # every piece claimed once; every staged strip (step 0's too with a returned image) complete
    total = tb["n_list0"] + tb["n_list1"] + (tb["n_local"] if copy_local else 0)
    assert sorted(claimed) == list(range(total))
    for h in range(TP):
        if h == 0 and not copy_local:
            continue
        _, strip0, nst, P = tb["steps"][h][:4]
        for lg in range(tb["LG"]):
            for pos in range(strip0, strip0 + nst):
                assert ctr.get((lg, tb["strip_list"][pos]), 0) == P, (h, lg, pos)


def test_in_loop_form_at_the_bench_shapes():
    """The TP=8 bench shapes with row strips take the in-loop form, their list-1
    pieces fit one K loop, and the first round reads only the local step and
    step 1 (bf16 all-gather: only the local step)."""
    for M, N, K, sched, dtype, h1 in ((16384, 13312, 16384, "AG_ROT_A", "BF16_F32", 0),
                                      (8192, 13312, 16384, "AG_ROT_B", "E4M3_BF16", 1),
                                      (8192, 8192, 3584, "RS_TILE_A_ROT_C", "BF16_F32", 1)):
        tb = dg.dist_gemm_fused_tables(M, N, K, 1, 8, sched, dtype)
        assert tb["loop"] == 1
        assert tb["n_list0"] == sum(tb["steps"][h][4] for h in range(1, h1 + 1))
        assert all(tb["steps"][h][0] <= tb["loop_capacity"] for h in range(h1 + 1, 8))


def test_fused_tables_errors():
    with pytest.raises(dg.DistGemmError) as e:
        dg.dist_gemm_fused_tables(512, 512, 64, 1, 1, "MONOLITHIC", "BF16_F32")
    assert e.value.status == -3
    for kw in ({"queues": 4}, {"step_group": 0}, {"copy_ahead": 65}, {"copy_chunk": 4104}, {"n_wg": 12},
               {"shared_a": 2}):
        with pytest.raises(dg.DistGemmError) as e:
            dg.dist_gemm_fused_tables(512, 512, 64, 1, 2, "AG_ROT_A", "BF16_F32", **kw)
        assert e.value.status == -1, kw
