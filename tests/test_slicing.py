"""Invariants of the balanced split's slices and of the merge's reading of
partial rows, emulated on the CPU with the device formulas (decode_mfma.hip:
num_slices, slice_begin, slice_of; the (slice, slot) rows the decode writes
and the merge reads).

Units are (sequence, 16-token block) pairs laid end to end; slice x covers
units [floor(x U / n), floor((x+1) U / n)).  A sequence cut by slice edges
leaves one partial row per slice it touches: slot 1 of the slice where it
began, slot 0 of every later one; the merge reads exactly slices
slice_of(first unit) .. slice_of(last unit).
"""
import numpy as np
import pytest


def num_slices(U, wgs):
    return min(U, wgs)


def slice_begin(x, U, n):
    return x * U // n


def slice_of(u, U, n):
    return ((u + 1) * n + U - 1) // U - 1


def rows_written(starts, U, n):
    """{(slice, slot): sequence} for every partial row the decode writes."""
    rows = {}
    for x in range(n):
        u0, u1 = slice_begin(x, U, n), slice_begin(x + 1, U, n)
        for b in range(len(starts) - 1):
            s, e = starts[b], starts[b + 1]
            if e <= u0 or s >= u1 or s == e:
                continue
            whole = s >= u0 and e <= u1
            if not whole:
                slot = 0 if s < u0 else 1
                assert (x, slot) not in rows, "two sequences share a partial row"
                rows[(x, slot)] = b
    return rows


@pytest.mark.parametrize("seed", range(16))
def test_slices_cover_units_once_and_the_merge_reads_exactly_the_written_rows(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 5, 64, 300]))
    lens = rng.integers(0, 5000, size=B)
    lens[rng.random(B) < 0.2] = 0
    nblk = -(-lens // 16)
    starts = np.concatenate([[0], np.cumsum(nblk)]).astype(int)
    U = int(starts[-1])
    if U == 0:
        return
    for wgs in (1, 3, 64, 256, 384, 2048, U + 7):
        n = num_slices(U, wgs)
        edges = [slice_begin(x, U, n) for x in range(n + 1)]
        assert edges[0] == 0 and edges[-1] == U
        assert all(edges[x + 1] > edges[x] for x in range(n)), "an empty slice"
        for u in set([0, U - 1] + list(rng.integers(0, U, size=50))):
            x = slice_of(u, U, n)
            assert edges[x] <= u < edges[x + 1]
        rows = rows_written(list(starts), U, n)
        read = {}
        for b in range(B):
            s, e = starts[b], starts[b + 1]
            if s == e:
                continue
            wf, wl = slice_of(s, U, n), slice_of(e - 1, U, n)
            if wf == wl:
                continue                        # written whole by its slice
            for w in range(wf, wl + 1):
                key = (w, 1 if w == wf else 0)
                read[key] = b
        assert read == rows, "the merge reads a row no slice wrote, or misses one"


def test_floor_edges_leave_empty_slices_when_slices_outnumber_units():
    """Why num_slices clamps to U: with more slices than units, floor edges
    leave empty slices between the parts of one sequence; they write no row,
    so a merge over wf..wl would read rows no slice of this call wrote."""
    U, n = 3, 8
    edges = [slice_begin(x, U, n) for x in range(n + 1)]
    empty = [x for x in range(n) if edges[x] == edges[x + 1]]
    assert empty == [0, 1, 3, 4, 6]
    wf, wl = slice_of(0, U, n), slice_of(U - 1, U, n)
    assert (wf, wl) == (2, 7) and set(range(wf, wl + 1)) & set(empty) == {3, 4, 6}


def test_first_slice_of_a_sequence_must_be_the_last_of_equal_edges():
    """With empty slices, the slice that holds unit u is the LAST x whose
    edge is <= u (what slice_of computes).  The plain inverse floor(u n / U)
    lands on an empty slice in front of it; a merge starting there would read
    slot 1 of a row nobody wrote and slot 0 of the slice where the decode
    wrote slot 1."""
    U, n = 3, 8
    s = 0
    naive = s * n // U
    assert naive == 0 and slice_begin(naive, U, n) == slice_begin(naive + 1, U, n)   # empty
    assert slice_of(s, U, n) == 2
    rows = rows_written([0, 3], U, n)
    assert (naive, 1) not in rows and (2, 1) in rows and (2, 0) not in rows
