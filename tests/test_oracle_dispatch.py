"""Pins for the oracle's rank-major dispatch.

Against library routines (np.bincount, np.cumsum, np.argsort(kind="stable")),
against invariants (every valid pair placed once, row_src inverts dst_row,
disjoint covering segments, source independence) and against a layout worked
out by hand (tests/golden/dispatch_hand_example.txt).
"""
import os

import numpy as np
import pytest

from oracle import layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_ids(rng, S, T_s, k, E, p_drop=0.0):
    ids = np.stack([np.stack([rng.choice(E, k, replace=False) for _ in range(T_s)])
                    for _ in range(S)]).astype(np.int32) if T_s else np.zeros((S, 0, k), np.int32)
    if p_drop:
        ids[rng.random(ids.shape) < p_drop] = -1
    return ids


@pytest.mark.parametrize("S,T_s,k,E,p_drop", [(2, 5, 2, 4, 0.0), (8, 16, 8, 32, 0.0),
                                              (3, 7, 3, 5, 0.3), (4, 0, 2, 4, 0.0)])
def test_matches_library_counting_sort(S, T_s, k, E, p_drop):
    rng = np.random.default_rng(S * 100 + T_s)
    ids = _random_ids(rng, S, T_s, k, E, p_drop)
    r = layer.dispatch(ids, E)
    seg = T_s * k
    for s in range(S):
        flat = ids[s].reshape(-1)
        valid = flat >= 0
        cnt = np.bincount(flat[valid], minlength=E)
        assert np.array_equal(r["cnt"][s], cnt)
        assert np.array_equal(r["off"][s], np.concatenate([[0], np.cumsum(cnt)[:-1]]))
        # stable sort of this source's valid pairs by expert = their window order
        order = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
        placed = r["dst_row"][s].reshape(-1)
        assert np.array_equal(placed[order], s * seg + np.arange(len(order)))
        assert np.all(placed[~valid] == -1)


def test_invariants():
    rng = np.random.default_rng(7)
    S, T_s, k, E = 8, 16, 8, 32
    ids = _random_ids(rng, S, T_s, k, E, 0.1)
    r = layer.dispatch(ids, E)
    valid = ids >= 0
    assert r["cnt"].sum() == valid.sum()
    dst = r["dst_row"][valid]
    assert len(np.unique(dst)) == len(dst)            # each pair placed once, no collisions
    flat_idx = np.arange(ids.size).reshape(ids.shape)[valid]
    assert np.array_equal(r["row_src"][dst], flat_idx)  # row_src inverts dst_row
    assert np.sum(r["row_src"] >= 0) == valid.sum()
    rows = layer.expert_rows(r["cnt"], r["off"], T_s, k)
    allrows = np.concatenate(rows)
    assert np.array_equal(np.sort(allrows), np.sort(dst))   # expert windows cover exactly
    for e, rr in enumerate(rows):
        src = r["row_src"][rr]
        assert np.all(ids.reshape(-1)[src] == e)
        assert np.all(np.diff(src) > 0)               # source-major, then pair order


def test_source_independence():
    """A source's segment depends on its own ids only (no metadata exchange)."""
    rng = np.random.default_rng(8)
    ids = _random_ids(rng, 4, 6, 3, 6)
    r1 = layer.dispatch(ids, 6)
    ids2 = ids.copy()
    ids2[1:] = _random_ids(rng, 3, 6, 3, 6)
    r2 = layer.dispatch(ids2, 6)
    assert np.array_equal(r1["cnt"][0], r2["cnt"][0])
    assert np.array_equal(r1["off"][0], r2["off"][0])
    assert np.array_equal(r1["dst_row"][0], r2["dst_row"][0])
    assert np.array_equal(r1["row_src"][:18], r2["row_src"][:18])


def test_degenerate_cases():
    # all pairs to one expert
    ids = np.zeros((2, 3, 1), np.int32)
    r = layer.dispatch(ids, 4)
    assert r["cnt"].tolist() == [[3, 0, 0, 0], [3, 0, 0, 0]]
    assert r["dst_row"].reshape(-1).tolist() == [0, 1, 2, 3, 4, 5]
    # nothing routed here
    r = layer.dispatch(np.full((2, 2, 2), -1, np.int32), 3)
    assert r["cnt"].sum() == 0 and np.all(r["row_src"] == -1)
    with pytest.raises(ValueError):
        layer.dispatch(np.array([[[5]]], np.int32), 4)


def _read_golden(path):
    sec, cur = {}, None
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            cur = line[:-1]
            sec[cur] = []
        else:
            sec[cur].append([int(v) for v in line.split()])
    return sec


def test_hand_worked_example():
    g = _read_golden(os.path.join(GOLDEN, "dispatch_hand_example.txt"))
    S, T_s, k, E = g["shape"][0]
    ids = np.array(g["ids"], dtype=np.int32).reshape(S, T_s, k)
    r = layer.dispatch(ids, E)
    assert r["cnt"].tolist() == g["cnt"]
    assert r["off"].tolist() == g["off"]
    assert r["dst_row"].reshape(S, T_s * k).tolist() == g["dst_row"]
    assert r["row_src"].tolist() == g["row_src"][0]
    rows = layer.expert_rows(r["cnt"], r["off"], T_s, k)
    assert [x.tolist() for x in rows] == [row[1:] if row[0] else [] for row in g["expert_rows"]]
