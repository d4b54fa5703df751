"""Host-side pieces of bench.py that need no GPU."""

import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


class _Lists:
    """Stands in for a plan: route_views returns fixed CPU counts and lists."""

    def __init__(self, counts, lists):
        self.counts, self.lists = counts, lists

    def route_views(self, ws):
        return self.counts, self.lists


def _case():
    nb = 40  # two groups of 32 key blocks, the second holding 8
    counts = torch.zeros(1, 1, nb, dtype=torch.int32)
    lists = torch.full((1, 1, nb, nb), 7, dtype=torch.int32)  # entries past the count are ignored
    counts[0, 0, 0] = nb
    lists[0, 0, 0] = torch.arange(nb)
    counts[0, 0, 1] = 32
    lists[0, 0, 1, :32] = torch.arange(32)
    counts[0, 0, 2] = 1
    lists[0, 0, 2, 0] = 5
    return _Lists(counts, lists)


@pytest.mark.parametrize("D,centroid,half_tiles", [
    # block 0: dense row, 80 exact half tiles, no centroids
    # block 1: the whole first group, 64 exact + the second group's centroid tile
    # block 2: one block, 2 exact + both centroid tiles
    # blocks 3..39: nothing selected, both centroid tiles each
    (128, True, 80 + 64 + 1 + 2 + 2 + 37 * 2),
    (64, True, 80 + 64 + 1 + 2 + 2 + 37 * 2),
    (128, False, 80 + 64 + 2),
])
def test_attend_mfma_count_by_hand(D, centroid, half_tiles):
    # two waves per query block, D/8 MFMAs per wave and half tile
    assert bench.attend_mfma_count(_case(), None, D, centroid=centroid) == 2 * half_tiles * (D // 8)


def test_attend_mfma_count_fully_selected_groups_need_no_centroid():
    nb = 64
    counts = torch.full((1, 2, nb), 32, dtype=torch.int32)
    lists = torch.zeros(1, 2, nb, nb, dtype=torch.int32)
    lists[0, 0, :, :32] = torch.arange(32)        # head 0: first group whole
    lists[0, 1, :, :32] = torch.arange(32, 64)    # head 1: second group whole
    n = bench.attend_mfma_count(_Lists(counts, lists), None, 128)
    assert n == 2 * (2 * nb * (2 * 32 + 1)) * 16
