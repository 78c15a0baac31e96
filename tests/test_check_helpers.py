"""CPU checks of the parity helper itself: a decode whose selection differs
from the oracle's inside the tie band must still have its output checked,
against the oracle's attention over the selection it made."""

import numpy as np
import pytest

import oracle
from gpu_cases import OracleSrc, check_decode


def _tied_case():
    # one head, S = 6, d = D = 2; tokens 2 and 4 have identical keys, so their
    # scores tie exactly at the k-th place (k = 2: token 0, then 2 or 4)
    P = np.eye(2)[None]
    q = np.array([[[1.0, 0.5]]])
    keys = np.array([[3.0, 0.0], [-1.0, 0.0], [1.0, 1.0], [0.0, -2.0], [1.0, 1.0], [-3.0, 1.0]])
    v = np.arange(12, dtype=np.float64).reshape(6, 2) ** 1.5
    slab = keys[None, None]
    rest = np.zeros((1, 1, 6, 0))
    vv = v[None, None]
    return q, P, slab, rest, vv


def test_swapped_pair_output_is_checked():
    q, P, slab, rest, vv = _tied_case()
    ref_out, ref_idx, ref_s = oracle.decode(q, slab, rest, vv, P, 2, "f64")
    assert ref_idx[0, 0].tolist() == [0, 2]  # the lower index wins the tie
    src = OracleSrc(q, slab, rest, vv, P)
    other = np.array([[[0, 4]]])  # also valid: token 4 ties with token 2
    good = oracle.attend_indices(q, slab, rest, vv, P, other, "f64")
    n_band, n_swap, worst = check_decode("f32", 2, good, other, ref_out, ref_idx, ref_s,
                                         [(0, 0)], src)
    assert (n_band, n_swap) == (1, 1) and worst <= 1e-12
    # token 4's value row differs from token 2's, so the oracle's own output is
    # wrong for the swapped set and must be rejected
    assert not np.allclose(good, ref_out)
    with pytest.raises(AssertionError, match="output error"):
        check_decode("f32", 2, ref_out, other, ref_out, ref_idx, ref_s, [(0, 0)], src)


def test_swap_outside_the_band_is_rejected():
    q, P, slab, rest, vv = _tied_case()
    ref_out, ref_idx, ref_s = oracle.decode(q, slab, rest, vv, P, 2, "f64")
    src = OracleSrc(q, slab, rest, vv, P)
    wrong = np.array([[[0, 1]]])  # token 1 scores far below the k-th place
    out = oracle.attend_indices(q, slab, rest, vv, P, wrong, "f64")
    with pytest.raises(AssertionError, match="invalid near-tie set"):
        check_decode("f32", 2, out, wrong, ref_out, ref_idx, ref_s, [(0, 0)], src)
