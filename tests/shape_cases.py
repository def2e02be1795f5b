"""Launch-shape cases shared by the forward and backward GPU parity tests.

SMALL: multi-tile problems with ragged tails over the launch-shape space
(chunks per head row 1..64 incl. non powers of two, L*P from 1 to 64, fp32 and
bf16 value, 2D and 3D with rows of up to 64 chunks, batch > 1, Lq a multiple
of no tile count).

STAGED: launches of >= 65536 (query, head) tiles: levels that fit the LDS
budget of the staged forward kernel or not, fp32/bf16, D from 4 to 64
channels, 2D/3D, query counts that leave ragged workgroups and waves, and a 2D
launch that the direct kernel takes with several tiles per wave.
"""

SMALL = [
    # dims, dtype, N, shapes, Lq, M, D, P
    (2, "f32", 2, ((20, 33), (10, 17), (5, 9), (3, 5)), 301, 8, 32, 4),
    (2, "bf16", 3, ((20, 33), (10, 17), (5, 9), (3, 5)), 257, 8, 32, 4),
    (2, "f32", 1, ((16, 16),), 67, 2, 8, 4),
    (2, "f32", 2, ((7, 9), (4, 5)), 33, 3, 4, 1),           # L*P = 2, D*4 = 16 B
    (2, "f32", 1, ((7, 9),), 45, 5, 12, 1),                 # L*P = 1, 3 chunks
    (2, "f32", 2, ((9, 11), (5, 6), (3, 3)), 29, 4, 64, 8),  # L*P = 24
    (2, "bf16", 2, ((9, 11), (5, 6)), 41, 2, 24, 32),       # L*P = 64, 3 chunks
    (2, "f32", 1, ((6, 10),) * 16, 13, 1, 128, 4),          # L = 16, L*P = 64
    (2, "f32", 2, ((12, 7), (6, 4)), 50, 2, 256, 3),        # 64 chunks per row
    (2, "bf16", 1, ((12, 7), (6, 4)), 50, 3, 512, 5),       # bf16, 64 chunks
    (2, "f32", 3, ((5, 5), (3, 3), (2, 2)), 19, 6, 20, 5),  # L*P = 15, 5 chunks
    (3, "f32", 2, ((8, 8, 8), (4, 4, 4), (2, 2, 2)), 219, 4, 32, 4),
    (3, "bf16", 1, ((6, 7, 9), (3, 4, 5)), 111, 8, 32, 3),
    (3, "f32", 1, ((3, 5, 7),), 37, 3, 8, 7),
    # 3D head rows of 32 and 64 chunks (fp32 D = 128 and 256, bf16 D = 256):
    # the widest rows of the 16-wave (8-wave fused/pruned) direct blocks, and
    # the 4-wave blocks beyond them
    (3, "f32", 1, ((5, 6, 7), (3, 3, 4)), 77, 2, 128, 3),
    (3, "bf16", 2, ((4, 5, 6),), 45, 3, 256, 2),
    (3, "f32", 1, ((3, 4, 5), (2, 2, 2)), 29, 2, 256, 2),
]

STAGED = [
    # dims, dtype, N, shapes, Lq, M, D, P, layout
    (2, "f32", 2, ((60, 90), (30, 45), (15, 23), (8, 12)), 7191, 8, 32, 4, "pixel_centres"),
    (2, "f32", 2, ((60, 90), (30, 45), (15, 23), (8, 12)), 4103, 8, 32, 2, "random_refs"),
    (2, "bf16", 2, ((60, 90), (30, 45), (15, 23), (8, 12)), 7191, 8, 32, 4, "pixel_centres"),
    (2, "f32", 1, ((40, 40), (7, 9)), 9001, 8, 64, 4, "random_refs"),
    (2, "f32", 3, ((50, 50), (3, 5)), 4099, 6, 8, 8, "uniform"),
    (2, "f32", 1, ((300, 300),), 70001, 1, 4, 4, "uniform"),     # no level fits
    (3, "f32", 2, ((16, 16, 16), (8, 8, 8), (4, 4, 4)), 4672, 8, 32, 4, "pixel_centres"),
    (3, "bf16", 1, ((16, 16, 16), (8, 8, 8), (4, 4, 4)), 9000, 8, 32, 2, "random_refs"),
    # bf16, 64 channels, L*P = 8: the backward's de-duplicating workgroups
    # would not fit the LDS (8 tiles per wave), so it takes the direct path
    (3, "bf16", 1, ((16, 16, 16), (8, 8, 8)), 8300, 8, 64, 4, "random_refs"),
    # a level one pixel wide (the backward's x < W/2 window is empty) and an
    # odd width
    (2, "f32", 1, ((97, 1), (13, 3)), 16500, 4, 16, 4, "random_refs"),
    # head rows that are not a power of two of 16-byte chunks in the large
    # launches: 3 chunks of 4 lanes (fp32 D = 12, bf16 D = 24) and 12 chunks
    # of 16 lanes (fp32 D = 48), with the pixel-centre and random layouts
    (2, "f32", 2, ((60, 90), (30, 45), (15, 23), (8, 12)), 7191, 8, 12, 4, "pixel_centres"),
    (2, "f32", 2, ((60, 90), (30, 45), (15, 23), (8, 12)), 7191, 8, 48, 4, "pixel_centres"),
    (2, "bf16", 2, ((60, 90), (30, 45), (15, 23), (8, 12)), 7191, 8, 24, 4, "pixel_centres"),
    (2, "f32", 1, ((60, 90), (30, 45), (15, 23), (8, 12)), 9000, 8, 12, 4, "random_refs"),
    # L * P = 9, P = 3: four tiles and two point groups per wave, G does not
    # divide P, so the forward takes the direct kernel with several tiles per
    # wave
    (2, "f32", 1, ((60, 90), (30, 45), (15, 23)), 9000, 8, 32, 3, "random_refs"),
]
