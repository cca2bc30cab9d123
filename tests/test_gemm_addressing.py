"""CPU replay of the grouped GEMMs' tile walk and operand addressing.

The grouped GEMM kernels map every block of a grid sized from the buffer-row
bound to one (expert, m-tile, n-tile) from the device offsets, or to nothing,
and address the tile's A rows with 32-bit element offsets from a 64-bit base
at the tile's first row. This file rebuilds that walk in NumPy for whole grids
and checks, for shapes whose row buffers hold more than 2^32 elements:

  * every block maps to at most one tile, and the valid tiles cover each
    expert's rows exactly once per n-tile;
  * every A address a tile forms lies inside its expert's rows;
  * every 32-bit offset (row offset + K position) fits in 32 bits, while the
    former whole-buffer offset (buffer row * K) would not.

The GPU regression of the same shape is in test_gpu_edges.py.
"""
import numpy as np
import pytest

import combine_top_softmax_amd as moe

NUM_XCD = 8
U32 = 1 << 32


def tile_walk(off, bm, ntn, grid, m_major):
    """Blocks -> tiles exactly as the kernels' lookup does: per-expert m-tile
    counts, tiles numbered expert by expert, blocks dealt to the XCDs round
    robin (block b takes tile (b % 8) * q + b / 8). m_major: the forward and
    MX order inside an expert (all m-tiles of n-tile 0 first) or the
    row-tile order of the backward (n fastest)."""
    off = np.asarray(off, dtype=np.int64)
    rows = np.maximum(off[1:] - off[:-1], 0)
    mt = (rows + bm - 1) // bm
    incl = np.cumsum(mt)
    total = int(incl[-1]) * ntn if len(mt) else 0
    q = (total + NUM_XCD - 1) // NUM_XCD
    b = np.arange(grid, dtype=np.int64)
    slot = b // NUM_XCD
    L = (b % NUM_XCD) * q + slot
    valid = (slot < q) & (L < total)
    L = L[valid]
    m_glob = L // ntn
    e = np.searchsorted(incl, m_glob, side="right")
    M = mt[e]
    mstart = incl[e] - M
    if m_major:
        li = L - mstart * ntn
        n = li // M
        m_in = li - n * M
    else:
        m_in = m_glob - mstart
        n = L - m_glob * ntn
    row0 = off[e] + m_in * bm
    return dict(block=b[valid], e=e, row0=row0, row_end=off[e + 1], row_begin=off[e], n=n,
                total=total)


def check_walk(off, Kdim, bm, ntn, grid, m_major, tile_rows=256, k_step=64, elems=8):
    w = tile_walk(off, bm, ntn, grid, m_major)
    assert len(w["block"]) == w["total"], "a tile without a block"
    # coverage: each (expert row, n-tile) exactly once
    E = len(off) - 1
    for e in range(E):
        sel = w["e"] == e
        n_rows = int(off[e + 1] - off[e])
        for nt in range(ntn):
            r0 = np.sort(w["row0"][sel & (w["n"] == nt)])
            want = np.arange(off[e], off[e + 1], bm) if n_rows > 0 else np.array([], np.int64)
            np.testing.assert_array_equal(r0, want)
    # addresses: tile row r -> clamped row offset from the tile base
    r = np.arange(tile_rows, dtype=np.int64)
    tr = np.minimum(r[None, :], (w["row_end"] - 1 - w["row0"])[:, None])
    a_off = tr * Kdim + (elems * 7)            # the last 16-byte chunk of a K step
    last = a_off + (Kdim - k_step)             # at the last K step
    assert int(last.max()) < U32, "a 32-bit in-tile offset wraps"
    addr = w["row0"][:, None] * Kdim + last    # element index in the buffer (64-bit)
    assert np.all(addr >= (w["row_begin"] * Kdim)[:, None])
    assert np.all(addr < (w["row_end"] * Kdim)[:, None])
    # the former offset from the buffer start would have wrapped
    return int((np.minimum(w["row0"][:, None] + r[None, :], w["row_end"][:, None] - 1) * Kdim).max())


def grid_blocks(rmax, E_L, bm, ntn):
    max_m = -(-rmax // bm) + E_L
    return -(-(max_m * ntn) // NUM_XCD) * NUM_XCD


# A dropless layer with every route kept (K = N = 8, one rank): 81,920 tokens
# give 655,360 buffer rows of d = 8192, 5.4e9 elements. The GPU regression
# test runs the same shape.
BIG = dict(T=81920, d=8192, N=8, K=8, F=128, ep_size=1, ep_rank=0, capacity=81920, dtype="bf16")


def test_big_buffer_shape_is_valid_and_past_2_32_elements():
    s = moe.MoeShape(**BIG)
    assert moe.moe_validate_shape(s) == 0
    assert s.rows == BIG["T"] * BIG["K"]
    assert s.rows * BIG["d"] > U32


@pytest.mark.parametrize("ragged", [False, True])
def test_up_gemm_addresses_stay_inside_their_expert(ragged):
    s = moe.MoeShape(**BIG)
    rows = s.rows
    E = BIG["N"]
    if ragged:
        # skewed expert loads summing to at most the buffer rows
        rng = np.random.default_rng(3)
        cnt = rng.integers(1, rows // E, size=E)
        cnt[2] = rows - int(cnt.sum() - cnt[2])
        cnt = np.maximum(cnt, 0)
        cnt[-1] += rows - int(cnt.sum())
    else:
        cnt = np.full(E, rows // E)
    off = np.concatenate([[0], np.cumsum(cnt)])
    assert off[-1] == rows
    ntn = -(-BIG["F"] // 128)
    grid = grid_blocks(rows, E, 256, ntn)
    old_max = check_walk(off, BIG["d"], 256, ntn, grid, m_major=True)
    assert old_max >= U32, "this shape must exercise offsets past 2^32"


def test_down_and_backward_row_tiles_stay_inside_their_expert():
    rows = BIG["T"] * BIG["K"]
    off = np.arange(0, rows + 1, rows // BIG["N"])
    # down GEMM (forward order, K = F, 256-wide n-tiles over d)
    ntn = -(-BIG["d"] // 256)
    check_walk(off, BIG["F"], 256, ntn, grid_blocks(rows, BIG["N"], 256, ntn), m_major=True)
    # backward dH (row tiles, K = d) and dX (K = 2F): n-tiles of 256
    for Kdim, n_out in ((BIG["d"], BIG["F"]), (2 * BIG["F"], BIG["d"])):
        ntn = -(-n_out // 256)
        check_walk(off, Kdim, 256, ntn, grid_blocks(rows, BIG["N"], 256, ntn), m_major=False)


def test_mx_scale_rows_stay_inside_their_expert():
    """MX up GEMM: qdata rows (Kdim bytes) and scale rows (Kdim/32 bytes) are
    both addressed from the tile's first row."""
    rows = BIG["T"] * BIG["K"]
    off = np.arange(0, rows + 1, rows // BIG["N"])
    ntn = -(-BIG["F"] // 128)
    grid = grid_blocks(rows, BIG["N"], 256, ntn)
    check_walk(off, BIG["d"], 256, ntn, grid, m_major=False, k_step=128, elems=16)
    check_walk(off, BIG["d"] // 32, 256, ntn, grid, m_major=False, k_step=4, elems=0)
