"""The multi-channel kernel's LDS slab staging, restated on the host.

The register-blocked kernel's matrix-core form stages each slab of input
channels (a 64 x 16 output tile plus its halo: the tile's own 64 columns of
every staged row, then a halo area of 8 floats per row) by DMA, either as
16-byte pixel groups (rows of whole vectors) or as dwords (any width). This
restates both index maps of `k2_multi.hip` (`slab_offsets`, and the dword
offsets of `is_k2_multi_mfma`) and checks on random geometries that they fill
the same LDS floats with the same input element, and that the dword map reads
zero exactly where the pixel lies outside the image. Host logic only.
"""
import random

TW, TH = 64, 16          # output tile columns and rows
MAIN_G, ALL_G = 16, 18   # 16-byte groups per staged row: the tile's own, and with the halo


def geometry(R, CS):
    P = (R - 1) // 2
    LH = TH + R - 1                          # staged rows per channel
    V4 = CS * LH * ALL_G                     # 16-byte vectors of a slab
    MAINV4 = CS * LH * MAIN_G                # the rows' own vectors come first
    rounds = ((V4 + 63) // 64 + 3) // 4      # 16-byte DMA rounds per wave
    return P, LH, V4, MAINV4, rounds


def vector_map(R, CS, x0, y0, H, W):
    """LDS float -> (channel, row, column) of the 16-byte path, None for 0."""
    P, LH, V4, MAINV4, rounds = geometry(R, CS)
    m = {}
    for q in range(rounds * 4 * 64):
        if q < MAINV4:
            c = q // (LH * MAIN_G)
            rem = q - c * LH * MAIN_G
            lrow = rem // MAIN_G
            g = 1 + rem - lrow * MAIN_G
        else:
            h = q - MAINV4
            c = h // (LH * 2)
            rem = h - c * LH * 2
            lrow = rem // 2
            g = ALL_G - 1 if rem & 1 else 0
        gy, gx = y0 - P + lrow, x0 - 4 + 4 * g
        inside = q < V4 and 0 <= gy < H and 0 <= gx < W
        for e in range(4):
            m[q * 4 + e] = (c, gy, gx + e) if inside else None
    return m


def dword_map(R, CS, x0, y0, H, W):
    """LDS float -> (channel, row, column) of the dword path, None for 0."""
    P, LH, V4, MAINV4, rounds = geometry(R, CS)
    main = CS * LH                            # one operation per staged row
    halo = (CS * LH * 8 + 63) // 64           # the halo area in pieces of 64 floats
    drounds = (main + halo + 3) // 4
    assert drounds * 4 * 16 <= rounds * 4 * 64, "the dword DMA stays in the pixel area"
    m = {}
    for ins in range(drounds * 4):
        for lane in range(64):
            c, lrow, gx = 0, 0, -1
            if ins < main:
                c, lrow = divmod(ins, LH)
                gx = x0 + lane
            else:
                h = (ins - main) * 64 + lane
                if h < CS * LH * 8:
                    crow, j8 = h >> 3, h & 7
                    c, lrow = divmod(crow, LH)
                    gx = x0 - 4 + j8 if j8 < 4 else x0 + TW + j8 - 4
            gy = y0 - P + lrow
            m[ins * 64 + lane] = (c, gy, gx) if (0 <= gx < W and 0 <= gy < H) else None
    return m


def wanted(R, CS, x0, y0, H, W, f):
    """What LDS float f of a slab must hold: its staged row and column."""
    P, LH, V4, MAINV4, rounds = geometry(R, CS)
    if f < MAINV4 * 4:
        crow, col = divmod(f, 64)
        gx = x0 + col
    else:
        crow, j8 = divmod(f - MAINV4 * 4, 8)
        gx = x0 - 4 + j8 if j8 < 4 else x0 + TW + j8 - 4
    c, lrow = divmod(crow, LH)
    gy = y0 - P + lrow
    return (c, gy, gx) if (0 <= gx < W and 0 <= gy < H) else None


def test_dword_and_vector_slab_maps_agree():
    rng = random.Random(1)
    for _ in range(400):
        R, CS = rng.choice([3, 5, 7]), rng.choice([1, 2])
        W, H = rng.randint(1, 300), rng.randint(1, 100)
        x0 = rng.randrange(0, (W + TW - 1) // TW) * TW
        y0 = rng.randrange(0, (H + TH - 1) // TH) * TH
        V4 = geometry(R, CS)[2]
        d = dword_map(R, CS, x0, y0, H, W)
        for f in range(V4 * 4):
            assert d[f] == wanted(R, CS, x0, y0, H, W, f), (R, CS, W, H, x0, y0, f)
        if W % 4 == 0:
            v = vector_map(R, CS, x0, y0, H, W)
            for f in range(V4 * 4):
                assert v[f] == d[f], (R, CS, W, H, x0, y0, f)
