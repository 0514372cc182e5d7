"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""

import numpy as np
import pytest

import oracle.attention as ref
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(ref)


def test_kv_head_map_is_contiguous():
    # the gate program's T2 map, checked on its own numbers
    assert list(ref.kv_head(np.arange(4), 4, 2)) == [0, 0, 1, 1]
    assert list(ref.kv_head(np.arange(128), 128, 16)[::8]) == list(range(16))
    with pytest.raises(ValueError):
        ref.kv_head(0, 6, 4)


def test_visible_pair_counts_closed_form():
    # |vis(i)| = min(i+1, W) + min(NS, max(0, i-W+1)) for a causal window,
    # summed over rows; i+1 without a window.
    for S, W, NS in [(50, 0, 0), (50, 7, 0), (50, 7, 3), (50, 7, 12), (50, 60, 5), (33, 1, 1)]:
        want = 0
        for i in range(S):
            if W == 0:
                want += i + 1
            else:
                want += min(i + 1, W) + min(NS, max(0, i - W + 1))
        assert ref.visible_pairs_per_head(S, True, W, NS) == want
