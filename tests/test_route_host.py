"""CPU replay of the two-kernel route's column sums (k_assign_scan): for every
shape the launcher sends there, the N * G threads of a block cover each
(expert, tile) histogram entry exactly once and index only the block's 256
partial-sum slots. Mirrors the launch rule and thread mapping in route.hip."""
import numpy as np
import pytest

FUSED_SCAN_MAX = 16384


def fused(N, ntiles):
    return N <= 256 and ntiles <= 256 and N * ntiles <= FUSED_SCAN_MAX


def group_width(N):
    G = 1
    while G < 64 and 2 * G * N <= 256:
        G *= 2
    return G


def covered(N, ntiles):
    G = group_width(N)
    hits = np.zeros((N, ntiles), np.int64)
    slots = set()
    for tid in range(256):
        ex, q = tid // G, tid % G
        if ex < N:
            slots.add(ex * G + q)
            hits[ex, q::G] += 1
    # the reduction reads slots ex * G + j, j < G, for every ex < N
    need = {ex * G + j for ex in range(N) for j in range(G)}
    return hits, need, slots


@pytest.mark.parametrize("N", [1, 2, 3, 5, 31, 32, 64, 65, 100, 127, 128, 129, 200, 255, 256])
def test_every_histogram_entry_is_summed_once(N):
    for ntiles in sorted({1, 2, 7, 63, 64, 65, 128, 255, 256, FUSED_SCAN_MAX // N}):
        if not (1 <= ntiles and fused(N, ntiles)):
            continue
        hits, need, slots = covered(N, ntiles)
        assert np.all(hits == 1), (N, ntiles)
        assert need <= slots and max(need) < 256, (N, ntiles)
        assert -(-ntiles // group_width(N)) <= 128   # column loads per thread


def test_launch_rule_sends_wide_or_long_maps_to_three_kernels():
    assert not fused(257, 1) and not fused(64, 257) and not fused(128, 129)
    assert fused(256, 64) and fused(64, 256) and fused(1, 256)
