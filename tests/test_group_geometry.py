"""Where the query groups sit in space: G consecutive tokens of the latent grid in Morton or cube order.

The DSV explainer (gist.science, hi edition, technical summary §2.B) groups 3D-adjacent queries, with
2x2x2 cubes as its example.  Here a group is G (64 or 128) consecutive tokens in Morton order.  These tests
measure, on the five workload grids, how many groups are one aligned box (4x4x4 for G = 64, 4x4x8 for
G = 128 -- each a union of whole aligned 2x2x2 cubes), how far the others spread, and how many hold cells
of the partial edge rows that a side not divisible by 4 leaves (45 rows at 57.6k tokens, 125 columns at
520k).  The cube order (the workloads' order="cubes" option) puts every whole aligned box first, so each of
its groups is one box, and the partial edge cells after them.  The counts are exact properties of the
orders; they are pinned so that a change of either order shows here.
"""
import numpy as np
import pytest

import synth


def geometry(grid, G, order="morton"):
    c = synth.morton_order(grid) if order == "morton" else synth.cube_order(grid, G)
    ng = len(c) // G
    cg = c[: ng * G].reshape(ng, G, 3)
    lo, hi = cg.min(1), cg.max(1)
    ext = hi - lo + 1
    box = ext.prod(1) == G                                        # the group fills its bounding box
    aligned = box & np.all(lo % ext == 0, axis=1)                 # ... and that box sits on the grid's own tiling
    cube = cg // 2                                                # the aligned 2x2x2 cube of each cell
    key = (cube[..., 0] * grid[1] + cube[..., 1]) * grid[2] + cube[..., 2]
    union = np.array([np.all(np.unique(k, return_counts=True)[1] == 8) for k in key])
    full = np.array([(n // 4) * 4 for n in grid])
    edge = np.any(cg >= full, axis=2).any(1)                      # holds a cell of a partial edge row
    return {"groups": ng, "aligned_boxes": int(aligned.sum()), "unions_of_2cubes": int(union.sum()),
            "edge_groups": int(edge.sum()), "max_extent": [int(v) for v in ext.max(0)],
            "max_box_cells": int(ext.prod(1).max()), "box_shapes": sorted({tuple(int(v) for v in e) for e in ext[aligned]})}


# workload: (groups, aligned boxes, unions of 2x2x2 cubes, groups with partial-edge cells, max bounding-box cells)
EXPECTED = {
    1: (16, 16, 16, 0, 64),
    2: (128, 128, 128, 0, 64),
    3: (900, 840, 860, 40, 240),
    4: (1024, 1024, 1024, 0, 128),
    5: (8125, 7865, 7865, 260, 240),
}


@pytest.mark.parametrize("wid", sorted(EXPECTED))
def test_morton_groups(wid):
    w = synth.workload(wid)
    g = geometry(w.grid, w.group)
    print(f"GROUPS {w.name} grid={w.grid} G={w.group} {g}")
    assert (g["groups"], g["aligned_boxes"], g["unions_of_2cubes"], g["edge_groups"], g["max_box_cells"]) == \
        EXPECTED[wid]
    # every aligned group is one cube-tiled box: 4x4x4, or two of them along one axis for G = 128
    shapes = {64: {(4, 4, 4)}, 128: {(4, 4, 8), (4, 8, 4), (8, 4, 4)}}[w.group]
    assert set(g["box_shapes"]) <= shapes
    if all(n % 4 == 0 for n in w.grid):
        assert g["aligned_boxes"] == g["groups"]     # sides divisible by 4: every group is one aligned box


# the same counts in cube order: every group one aligned box; the partial edge rows form flat boxes
EXPECTED_CUBES = {
    1: (16, 16, 16, 0, 64),
    2: (128, 128, 128, 0, 64),
    3: (900, 900, 880, 20, 64),
    4: (1024, 1024, 1024, 0, 128),
    5: (8125, 8125, 8060, 65, 64),
}


@pytest.mark.parametrize("wid", sorted(EXPECTED_CUBES))
def test_cube_order_groups(wid):
    w = synth.workload(wid)
    g = geometry(w.grid, w.group, "cubes")
    print(f"GROUPS {w.name} order=cubes grid={w.grid} G={w.group} {g}")
    assert (g["groups"], g["aligned_boxes"], g["unions_of_2cubes"], g["edge_groups"], g["max_box_cells"]) == \
        EXPECTED_CUBES[wid]
    # the whole-box groups are the cube box itself; the groups of the partial edge cells are flat aligned boxes
    assert tuple(synth.cube_box(w.group)) in set(g["box_shapes"])
    assert g["unions_of_2cubes"] == g["groups"] - g["edge_groups"]


def test_cube_order_is_a_permutation_with_whole_boxes_first():
    grid, G = (8, 10, 12), 64
    c = synth.cube_order(grid, G)
    assert sorted(map(tuple, c.tolist())) == sorted(map(tuple, synth.morton_order(grid).tolist()))
    # 2 x 2 x 3 whole 4x4x4 boxes (y 0..7), each one group, then the 192 cells of rows y = 8, 9
    whole = c[: 12 * 64].reshape(12, 64, 3)
    lo = whole.min(1)
    assert np.all(whole.max(1) - lo == 3) and np.all(lo % 4 == 0)
    assert len({tuple(v) for v in lo.tolist()}) == 12
    assert np.all(c[12 * 64:, 1] >= 8)


def test_geometry_measure_on_a_hand_case():
    # a 4x4x8 grid in Morton order: 64-token groups are the two aligned 4x4x4 cubes, x = 0..3 and x = 4..7
    g = geometry((4, 4, 8), 64)
    assert g == {"groups": 2, "aligned_boxes": 2, "unions_of_2cubes": 2, "edge_groups": 0, "max_extent": [4, 4, 4],
                 "max_box_cells": 64, "box_shapes": [(4, 4, 4)]}
    # 8x5x4: in Morton order the cube t 0..3, y 0..3 comes first, then the 16 cells of row y = 4 beside it (a
    # cut-off cube), then the cube t 4..7: the second group is those 16 cells and 48 of the next cube, a
    # group spread over the whole 8x5x4 box and holding the partial row
    g = geometry((8, 5, 4), 64)
    assert (g["groups"], g["aligned_boxes"], g["edge_groups"], g["max_box_cells"]) == (2, 1, 1, 160)
    # the same grid in cube order: the two whole cubes first, then the 32 cells of row y = 4 (not a group)
    g = geometry((8, 5, 4), 64, "cubes")
    assert (g["groups"], g["aligned_boxes"], g["edge_groups"], g["max_box_cells"]) == (2, 2, 0, 64)
