"""fmha_check_seqlens on the device against the varlen contract, checked by
a brute-force loop on the host ("Adds variable sequence lengths to the Hopper
CuTe DSL FMHA example", section Interface: cumulative int32 lengths starting
at 0, with a bound on the longest sequence)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fmha():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import split_kv_flash_fmha_amd as m
    return m


def expected(cu, total, max_len):
    """1 + the first index at which the contract fails, else 0."""
    for b, c in enumerate(cu):
        bad = (b == 0 and c != 0)
        if b > 0:
            bad = bad or c < cu[b - 1] or c - cu[b - 1] > max_len
        if b == len(cu) - 1:
            bad = bad or c != total
        if bad:
            return b + 1
    return 0


CASES = [
    ([0, 3, 3, 10], 10, 7),      # valid, with an empty sequence
    ([1, 3, 10], 10, 9),         # first entry not 0
    ([0, 5, 4, 10], 10, 9),      # decrease
    ([0, 3, 12], 12, 8),         # a sequence longer than the bound
    ([0, 3, 10], 11, 9),         # last entry != total
    ([0], 0, 0),                 # no sequences
    ([5], 5, 9),                 # no sequences, bad first entry
    ([0, 2 ** 31 - 1, -5], 0, 2 ** 31 - 1),  # extreme values: no overflow in the differences
]


@pytest.mark.parametrize("cu,total,max_len", CASES)
def test_small_cases(fmha, cu, total, max_len):
    sys.__stderr__.write(f"[gpu-case] check_seqlens {cu} total={total} max={max_len}\n")
    t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    assert fmha.check_seqlens(t, total, max_len) == expected(cu, total, max_len)


def test_many_sequences(fmha):
    # beyond one entry per thread; a fault planted late, then an earlier one
    rng = np.random.default_rng(16)
    lens = rng.integers(0, 700, size=5000)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total, max_len = int(cu[-1]), int(lens.max())
    sys.__stderr__.write("[gpu-case] check_seqlens 5000 sequences\n")
    t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    assert fmha.check_seqlens(t, total, max_len) == 0
    assert fmha.check_seqlens(t, total, max_len - 1) == expected(list(cu), total, max_len - 1) > 0
    bad = cu.copy()
    bad[4321] = bad[4320] - 1
    t = torch.tensor(bad, dtype=torch.int32, device="cuda")
    assert fmha.check_seqlens(t, total, 10 ** 6) == 4322
    bad[17] = bad[16] - 1
    t = torch.tensor(bad, dtype=torch.int32, device="cuda")
    assert fmha.check_seqlens(t, total, 10 ** 6) == 18


def test_rejects_bad_arguments(fmha):
    with pytest.raises(ValueError):
        fmha.check_seqlens(torch.zeros(3, dtype=torch.int64, device="cuda"), 0, 0)
    with pytest.raises(ValueError):
        fmha.check_seqlens(torch.zeros(3, dtype=torch.int32, device="cuda"), -1, 0)
