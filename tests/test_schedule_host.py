"""The attention kernel's work schedule, checked on the CPU through the
host-check library (the same header code the kernel and the merge kernel
run): every (item, key tile) unit of a call is run exactly once, every piece
of the last round has a partial slot of its own, and the merge reads exactly
an item's pieces in key order.  No GPU needed."""
import ctypes

import numpy as np
import pytest

from chunked_kv_cache_amd import ff

MAX_WG = 256
PIECE_COST = 6          # tiles charged per piece by the level split


@pytest.fixture(scope="module")
def lib():
    L = ff.load(ff.HOSTCHECK_PATH)
    L.ffstub_schedule_pieces.restype = ctypes.c_int
    L.ffstub_schedule_pieces.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_int]
    L.ffstub_merge_slots.restype = ctypes.c_int
    L.ffstub_merge_slots.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_int]
    return L


def pieces(L, n_items, ntiles, n_wg):
    cap = n_items * n_wg + 4 * n_wg
    out = np.zeros((cap, 5), dtype=np.int32)
    n = L.ffstub_schedule_pieces(n_items, ntiles, n_wg, out.ctypes.data, cap)
    assert n >= 0
    return out[:n]


def merge_slots(L, n_items, ntiles, n_wg, x):
    cap = 4 * MAX_WG
    out = np.zeros(cap, dtype=np.int32)
    n = L.ffstub_merge_slots(n_items, ntiles, n_wg, x, out.ctypes.data, cap)
    assert 0 <= n <= 2 * MAX_WG          # the merge kernel's LDS list holds 2 x 256 entries
    return out[:n]


SHAPES = [(n_items, nt, n_wg)
          for n_wg in (1, 3, 8, 37, 256)
          for n_items in (1, 2, 5, 12, 120, 228, 257, 264)
          for nt in (1, 2, 7, 64, 488)]


@pytest.mark.parametrize("n_items,ntiles,n_wg", SHAPES)
def test_schedule_covers_every_unit_once(lib, n_items, ntiles, n_wg):
    P = pieces(lib, n_items, ntiles, n_wg)
    cover = np.zeros((n_items, ntiles), dtype=np.int32)
    for g, item, tb, te, slot in P:
        assert 0 <= g < n_wg and 0 <= item < n_items and 0 <= tb < te <= ntiles
        cover[item, tb:te] += 1
    assert (cover == 1).all()
    full = n_items // n_wg
    # whole items of the full rounds write O directly; every last-round piece
    # has a slot of its own inside the 2 x n_wg partial region
    slots = P[:, 4]
    assert ((P[:, 1] < full * n_wg) == (slots < 0)).all()
    used = slots[slots >= 0]
    assert len(set(used.tolist())) == len(used)
    assert (used < 2 * n_wg).all()
    # pieces of a full-round item: one whole item per workgroup and round
    whole = P[slots < 0]
    assert (whole[:, 2] == 0).all() and (whole[:, 3] == ntiles).all()


@pytest.mark.parametrize("n_items,ntiles,n_wg", SHAPES)
def test_merge_reads_each_items_pieces_in_key_order(lib, n_items, ntiles, n_wg):
    P = pieces(lib, n_items, ntiles, n_wg)
    full, rem = n_items // n_wg, n_items % n_wg
    by_slot = {int(r[4]): r for r in P if r[4] >= 0}
    for x in range(rem):
        item = full * n_wg + x
        got = [s for s in merge_slots(lib, n_items, ntiles, n_wg, x) if s >= 0]
        written = sorted(int(r[4]) for r in P if r[1] == item)
        assert sorted(got) == written
        ranges = [(int(by_slot[s][2]), int(by_slot[s][3])) for s in got]
        assert ranges[0][0] == 0 and ranges[-1][1] == ntiles
        assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))


@pytest.mark.parametrize("n_items,ntiles", [(120, 488), (120, 513), (228, 488), (264, 1182), (258, 1182)])
def test_schedule_balance_on_the_workload_shapes(lib, n_items, ntiles):
    """480p (120 items of 512 queries x 488 or 513 tiles), 720p (264 items x
    1182 tiles) and a 256-query form (228 items): the busiest workgroup,
    counting kPieceCost tiles per piece, stays within 4% of the average."""
    P = pieces(lib, n_items, ntiles, 256)
    load = np.zeros(256)
    for g, item, tb, te, slot in P:
        load[g] += (te - tb) + (PIECE_COST if slot >= 0 else 0)
    assert load.max() <= 1.04 * load.mean()
