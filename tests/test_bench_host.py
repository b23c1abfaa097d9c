"""Host-side bookkeeping of bench.py: the count of half-block products the
forward kernel skips on key halves that are all pad (the issued FLOPs reported
beside the roofline), against a direct walk over the lists."""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def walk(pad_hi, counts, idx):
    """The kernel's rule, one list at a time: S of listed block k (k >= 1) is
    skipped when its upper half is pad; its PV when it is pad and the next
    listed block is pad too or there is none."""
    total = 0
    H, M = counts.shape
    for h in range(H):
        for i in range(M):
            lst = [int(x) for x in idx[h, i, :counts[h, i]]]
            for k, b in enumerate(lst):
                if not pad_hi[b]:
                    continue
                if k >= 1:
                    total += 1
                if k == len(lst) - 1 or pad_hi[lst[k + 1]]:
                    total += 1
    return total


def test_hand_example():
    # blocks 2 and 3 have pad upper halves
    pad_hi = torch.tensor([False, False, True, True])
    counts = torch.tensor([[4, 2, 1, 0]], dtype=torch.int32)
    idx = torch.zeros((1, 4, 4), dtype=torch.int32)
    idx[0, 0] = torch.tensor([0, 2, 3, 1])  # 2: S, PV (next is 3); 3: S only (next 1 is real)
    idx[0, 1, :2] = torch.tensor([2, 3])    # 2 first: S computed, PV skipped; 3: S, PV (last)
    idx[0, 2, :1] = torch.tensor([3])       # first and last: S computed, PV skipped
    # row 0: 2 + 1, row 1: 1 + 2, row 2: 1, row 3: empty
    assert bench.skipped_pair_products(pad_hi, counts, idx) == 7
    assert walk(pad_hi.numpy(), counts.numpy(), idx.numpy()) == 7


def test_random_lists_match_walk():
    rng = np.random.default_rng(3)
    for H, M in ((1, 1), (2, 7), (3, 33)):
        pad_hi = rng.random(M) < 0.35
        counts = rng.integers(0, M + 1, size=(H, M)).astype(np.int32)
        idx = np.zeros((H, M, M), dtype=np.int32)
        for h in range(H):
            for i in range(M):
                idx[h, i, :counts[h, i]] = np.sort(rng.choice(M, counts[h, i], replace=False))
        got = bench.skipped_pair_products(torch.from_numpy(pad_hi), torch.from_numpy(counts),
                                          torch.from_numpy(idx))
        assert got == walk(pad_hi, counts, idx)
