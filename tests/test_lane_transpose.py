"""CPU check of the decode kernel's 4 x 4 dword transpose across the four
16-lane rows of a wave (used when a quantization group is 32 or 64 K values,
so that each MFMA step holds one 32-deep sub-block of every column).

Row R of the wave holds, in registers d0..d3, the four dwords of K sub-block
R of its column (the GFX950_B lane load). After the transpose register j of
row R must hold dword R of sub-block j. The two lane-swap instructions are
emulated from their lane layout on gfx950, checked on the GPU with an
in-bounds probe (rows of 16 lanes):
  v_permlane32_swap(a, b) -> a' = [a0, a1, b0, b1], b' = [a2, a3, b2, b3]
  v_permlane16_swap(a, b) -> a' = [a0, b0, a2, b2], b' = [a1, b1, a3, b3]"""


def p32(a, b):
    return [a[0], a[1], b[0], b[1]], [a[2], a[3], b[2], b[3]]


def p16(a, b):
    return [a[0], b[0], a[2], b[2]], [a[1], b[1], a[3], b[3]]


def transpose(d):
    """d[j] = register j as a list over rows; the kernel's sequence."""
    d = list(d)
    d[0], d[2] = p32(d[0], d[2])
    d[1], d[3] = p32(d[1], d[3])
    d[0], d[1] = p16(d[0], d[1])
    d[2], d[3] = p16(d[2], d[3])
    return d


def test_transpose_of_sub_block_dwords():
    # value (sub-block s, dword j) placed where the lane load puts it: row s, register j
    d = [[(s, j) for s in range(4)] for j in range(4)]
    e = transpose(d)
    for j in range(4):
        for r in range(4):
            assert e[j][r] == (j, r), (j, r, e[j][r])
