"""Pins of the visit-order oracle (CPU): textbook Z-order sequences, a
hand-derived two-level example, the aligned-square property of the Z-order
curve, and invariants of the two tie-breaking rules."""
import numpy as np
import pytest

from oracle.order import query_order_oracle

# The Z-order (Morton) curve over a 4x4 grid, as raster indices i*4 + j: it
# visits the four 2x2 quadrants in the order (top-left, top-right,
# bottom-left, bottom-right), and each quadrant in the same pattern.
Z_ORDER_4x4 = [0, 1, 4, 5, 2, 3, 6, 7, 8, 9, 12, 13, 10, 11, 14, 15]


@pytest.mark.parametrize("level_major", [True, False])
def test_single_level_4x4_is_the_textbook_z_order(level_major):
    assert query_order_oracle([(4, 4)], level_major).tolist() == Z_ORDER_4x4


def test_single_level_2x2x2_and_first_octant_of_4x4x4():
    # x varies fastest, then y, then z: the 2x2x2 cube in raster order
    assert query_order_oracle([(2, 2, 2)], True).tolist() == list(range(8))
    # the first 8 entries of 4x4x4 are the corner cube {0,1}^3:
    # raster index (k*4 + i)*4 + j
    first = sorted(query_order_oracle([(4, 4, 4)], True)[:8].tolist())
    assert first == [0, 1, 4, 5, 16, 17, 20, 21]


def test_two_levels_by_hand():
    # Level 0 is 2x2 (pixels 0..3), level 1 is 1x1 (pixel 4).  On the 1024-cell
    # grid the 2x2 pixel centres 0.25 / 0.75 fall in cells 256 / 768 and the
    # 1x1 centre 0.5 in cell 512.  Keys (x bit b -> 2b, y bit b -> 2b+1):
    #   (y, x) = (256, 256): 0x30000   pixel 0
    #            (256, 768): 0x70000   pixel 1
    #            (768, 256): 0xB0000   pixel 2
    #            (768, 768): 0xF0000   pixel 3
    #            (512, 512): 0xC0000   pixel 4 (level 1)
    assert query_order_oracle([(2, 2), (1, 1)], False).tolist() == [0, 1, 2, 4, 3]
    assert query_order_oracle([(2, 2), (1, 1)], True).tolist() == [0, 1, 2, 3, 4]


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_power_of_two_grid_blocks_are_aligned_squares(k):
    # For a 2^k x 2^k level every aligned run of 4^s consecutive entries of a
    # Z-order is a 2^s x 2^s square at a multiple of 2^s.
    n = 1 << k
    order = query_order_oracle([(n, n)], True)
    for s in range(k + 1):
        side = 1 << s
        for b in range(0, n * n, side * side):
            block = order[b:b + side * side]
            i, j = block // n, block % n
            assert i.min() % side == 0 and j.min() % side == 0
            assert i.max() - i.min() == side - 1 and j.max() - j.min() == side - 1
            assert len(set(block.tolist())) == side * side


def test_rectangular_level_by_hand():
    # A 2x4 level (H=2, W=4): x cells 128, 384, 640, 896 (bits 7 | 8,7 | 9,7 |
    # 9,8,7) and y cells 256, 768 (bits 8 | 9,8).  Key bit 2b+1 carries y's
    # bit b, so y's bit 9 (key bit 19) is above all of x's bits (key bits <= 18):
    # row 0 comes entirely before row 1, and within a row the keys grow with x.
    assert query_order_oracle([(2, 4)], True).tolist() == list(range(8))
    # The transposed level (H=4, W=2): x cells 256, 768, y cells 128, 384, 640,
    # 896.  x's bit 9 (key bit 18) splits the columns before y's bit 8 (key
    # bit 17) splits the rows, and y's bit 9 (key bit 19) is on top: the order
    # is rows 0-1 column 0 ... as raster indices i*2 + j:
    #   keys (i, j): y bits at 2b+1, x bits at 2b
    #   (0,0) 2^15+2^16    (0,1) 2^15+2^16+2^18   (1,0) 2^15+2^17+2^16
    #   (1,1) 2^15+2^17+2^16+2^18  (2,0) 2^15+2^19+2^16  (2,1) 2^15+2^19+2^16+2^18
    #   (3,0) 2^15+2^19+2^17+2^16  (3,1) 2^15+2^19+2^17+2^16+2^18
    # sorted: (0,0) (1,0) (0,1) (1,1) (2,0) (3,0) (2,1) (3,1)
    assert query_order_oracle([(4, 2)], True).tolist() == [0, 2, 1, 3, 4, 6, 5, 7]


@pytest.mark.parametrize("shapes", [
    [(100, 150), (50, 75), (25, 38), (13, 19)],
    [(7, 1), (1, 9), (3, 3)],
    [(1, 1500), (2, 700)],          # wider than 1024 cells: ties by raster index
    [(16, 16, 16), (8, 8, 8), (5, 3, 7)],
])
def test_permutation_and_tie_rules(shapes):
    dims = len(shapes[0])
    sizes = [int(np.prod(s)) for s in shapes]
    starts = np.cumsum([0] + sizes)
    S = starts[-1]
    inter = query_order_oracle(shapes, False)
    major = query_order_oracle(shapes, True)
    for order in (inter, major):
        assert sorted(order.tolist()) == list(range(S))
    # level-major: levels appear one after another, each in the interleaved
    # order's relative sequence
    level_of = np.searchsorted(starts, np.arange(S), side="right") - 1
    assert (np.diff(level_of[major]) >= 0).all()
    for l in range(len(shapes)):
        assert (inter[level_of[inter] == l] == major[level_of[major] == l]).all()
    if dims == 2 and shapes[0] == (1, 1500):
        # a single-row level wider than the grid: raster order is preserved
        assert (major[:1500] == np.arange(1500)).all()


# ---- the order of queries given by one point each (data-dependent reference
# points): Morton key of the point's cell on a 2^16 (2D) or 2^10 (3D) grid,
# ties by query index.

from oracle.order import point_cells, points_order_oracle  # noqa: E402


def test_points_quadrant_centres_follow_the_z_pattern():
    # the four quadrant centres, given in a scrambled order: the Z pattern is
    # (x low, y low), (x high, y low), (x low, y high), (x high, y high)
    pts = np.array([[0.75, 0.75], [0.25, 0.75], [0.75, 0.25], [0.25, 0.25]], np.float32)
    assert points_order_oracle(pts).tolist() == [3, 2, 1, 0]
    # octant centres in 3D: x is the lowest key bit, then y, then z
    oct_ = np.array([[x, y, z] for z in (0.75, 0.25) for y in (0.75, 0.25) for x in (0.75, 0.25)],
                    np.float32)
    order = points_order_oracle(oct_)
    got = [tuple(oct_[i]) for i in order]
    want = [(x, y, z) for z in (0.25, 0.75) for y in (0.25, 0.75) for x in (0.25, 0.75)]
    assert got == want


@pytest.mark.parametrize("dims,k", [(2, 1), (2, 3), (2, 5), (3, 1), (3, 3)])
def test_points_order_of_pixel_centres_matches_the_pixel_order(dims, k):
    # a single 2^k-per-axis level: the pixel centres (j + 1/2) / 2^k lie in
    # cells j * 2^(B-k) + 2^(B-k-1), whose high bits are j, so both orders are
    # the Morton order of the pixels (computed independently: the pixel order
    # from its own 10-bit cells)
    e = 1 << k
    shape = (e,) * dims
    idx = np.arange(e ** dims)
    coords = []
    rest = idx
    for _ in range(dims):                  # x fastest
        coords.append(rest % e)
        rest = rest // e
    pts = np.stack([(c + 0.5) / e for c in coords], axis=1).astype(np.float32)
    assert points_order_oracle(pts).tolist() == query_order_oracle([shape], False).tolist()


def test_points_cells_clamp_and_nan():
    pts = np.array([[np.nan, 0.5], [-0.25, 1.0], [2.0, np.inf], [-np.inf, 0.999999]], np.float32)
    c = point_cells(pts)
    top = (1 << 16) - 1
    assert c.tolist() == [[0, 32768], [0, top], [top, top], [0, int(np.floor(np.float32(0.999999) * 65536))]]


def test_points_order_is_a_stable_sort_by_key():
    rng = np.random.default_rng(7)
    for dims in (2, 3):
        # clustered points with exact duplicates: ties go by query index
        pts = rng.random((500, dims)).astype(np.float32)
        pts[100:140] = pts[3]
        order = points_order_oracle(pts)
        assert sorted(order.tolist()) == list(range(500))
        cells = point_cells(pts)
        bits = 16 if dims == 2 else 10
        # key by explicit bit interleaving, written independently of morton_key
        def key(c):
            k = 0
            for b in range(bits):
                for d in range(dims):
                    k |= ((int(c[d]) >> b) & 1) << (dims * b + d)
            return k
        keys = [key(cells[i]) for i in order]
        assert all(a <= b for a, b in zip(keys, keys[1:]))
        for a, b, ka, kb in zip(order, order[1:], keys, keys[1:]):
            if ka == kb:
                assert a < b
