"""Host check of the LDS fragment-address identities the HIP kernels rely on.

`csrc/gdr_lds.h` stores bf16 tiles unpadded with an XOR swizzle of the 16-byte
pieces of each row (`swz`, `prow`, `soff`) and forms every fragment address from a
per-lane part and the fragment's tile-aligned offsets (`rk_lane`, `kc_lane`,
`kcs_lane`, `rks_lane`): one XOR per distinct offset instead of the swizzle per
read.  This test restates both forms (the functions below mirror the header's) and
checks, for every lane, tile width and swizzle kind the kernels use and every
aligned offset, that the decomposed address equals the swizzled one.  No GPU."""

import pytest


def swz(W, K, r):
    if W == 128:
        return (r ^ (r << 1)) & 15
    if W == 64 and K == 0:
        return 4 * ((r >> 1) & 1) + 2 * ((r & 1) ^ ((r >> 3) & 1)) + ((r >> 2) & 1)
    if W == 64:
        return r & 7
    return 0


def prow(W, r):
    return r ^ (((r >> 3) & 1) << 2) if W == 16 else r


def soff(W, K, r, c):
    return prow(W, r) * (2 * W) + (((c >> 3) ^ swz(W, K, r)) << 4) + ((c & 7) << 1)


def rk_lane(W, K, q, g):
    return prow(W, q) * 2 * W + ((g ^ swz(W, K, q)) << 4)


def kc_lane(W, K, q, g, d):
    rl = 8 * g + (q >> 2) + d
    return prow(W, rl) * 2 * W + 8 * (q & 1) + ((((q >> 1) & 1) ^ swz(W, K, rl)) << 4)


def kcs_lane(W, K, q, g):
    rl = 4 * g + (q >> 2)
    return prow(W, rl) * 2 * W + 8 * (q & 1) + ((((q >> 1) & 1) ^ swz(W, K, rl)) << 4)


def rks_lane(W, K, q, g):
    return prow(W, q) * 2 * W + 8 * (g & 1) + (((g >> 1) ^ swz(W, K, q)) << 4)


# (tile width in bf16 elements, swizzle kind, rows): the tiles of the recursion,
# gradient and output kernels (64 x D, D x D, D x 64, 64 x 64, 16-row slices, and
# the 64 x 16 dO slices)
TILES = [(128, 0, 128), (128, 0, 64), (128, 0, 16), (64, 0, 64), (64, 0, 128), (64, 1, 128), (64, 1, 16),
         (16, 0, 64)]


@pytest.mark.parametrize("W,K,rows", TILES, ids=[f"w{w}_k{k}_r{r}" for w, k, r in TILES])
def test_fragment_addresses(W, K, rows):
    for lane in range(64):
        q, g = lane & 15, lane >> 4
        if W >= 32:
            for r0 in range(0, rows, 16):
                for k0 in range(0, W, 32):
                    # row fragment: rows r0 + q, columns k0 + 8g .. +7
                    assert soff(W, K, r0 + q, k0 + 8 * g) == r0 * 2 * W + (rk_lane(W, K, q, g) ^ (2 * k0))
                    # split-K row fragment: columns k0 + 4g and k0 + 16 + 4g
                    L = rks_lane(W, K, q, g)
                    assert soff(W, K, r0 + q, k0 + 4 * g) == r0 * 2 * W + (L ^ (2 * k0))
                    assert soff(W, K, r0 + q, k0 + 16 + 4 * g) == r0 * 2 * W + (L ^ (2 * k0 + 32))
        for k0 in range(0, rows - 31, 32):
            for c0 in range(0, W, 16):
                c = c0 + 4 * (q & 3)
                # transposed fragment: rows k0 + 8g + q/4 and 4 below
                r = k0 + 8 * g + (q >> 2)
                assert soff(W, K, r, c) == k0 * 2 * W + (kc_lane(W, K, q, g, 0) ^ (2 * c0))
                assert soff(W, K, r + 4, c) == k0 * 2 * W + (kc_lane(W, K, q, g, 4) ^ (2 * c0))
                # split-K transposed fragment: rows k0 + 4g + q/4 and 16 below
                r = k0 + 4 * g + (q >> 2)
                L = kcs_lane(W, K, q, g)
                assert soff(W, K, r, c) == k0 * 2 * W + (L ^ (2 * c0))
                assert soff(W, K, r + 16, c) == (k0 + 16) * 2 * W + (L ^ (2 * c0))


@pytest.mark.parametrize("W,K,rows", TILES, ids=[f"w{w}_k{k}_r{r}" for w, k, r in TILES])
def test_swizzle_is_a_permutation(W, K, rows):
    # every (row, 16-byte piece) lands on a distinct slot of the tile
    pieces = W // 8
    slots = {soff(W, K, r, 8 * p) for r in range(rows) for p in range(pieces)}
    assert len(slots) == rows * pieces
    assert min(slots) == 0 and max(slots) == (rows * pieces - 1) * 16
