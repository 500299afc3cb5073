"""The comparison rules themselves (tests/parity.py), on constructed CPU cases: a legitimate alternative
selection on a near-tie token passes, a wrong expert does not, whatever the token's flag."""
import numpy as np
import pytest

import oracle
from tests.parity import check_routing


def _case():
    # token 0: clear top-2 {3, 1}; token 1: 2nd/3rd logits 5e-5 apart (flagged), so {0, 2} or {0, 4} are both a
    # top-2 within the gap
    l = np.array([[0.1, 2.0, -1.0, 3.0, 0.5],
                  [4.0, -2.0, 1.00005, -3.0, 1.0]])
    assert list(oracle.topk_flags(l, 2)) == [False, True]
    return l


def test_alternative_choice_on_a_flagged_token_passes():
    l = _case()
    idx = np.array([[3, 1], [0, 4]])  # token 1 takes the other side of its near-tie
    check_routing(idx, oracle.topk_weights(l, idx), l, 2)


@pytest.mark.parametrize("idx,why", [
    ([[3, 1], [0, 3]], "flagged token picks an expert far below its top-2"),
    ([[3, 0], [0, 2]], "unflagged token's set differs"),
    ([[3, 3], [0, 2]], "expert chosen twice"),
    ([[3, 1], [0, 7]], "expert out of range"),
])
def test_wrong_choices_fail(idx, why):
    l = _case()
    idx = np.array(idx)
    with pytest.raises(AssertionError):
        w = oracle.topk_weights(l, np.clip(idx, 0, 4))
        check_routing(idx, w, l, 2)
