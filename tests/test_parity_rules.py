"""CPU checks of the comparison rules in tests/parity.py themselves: codes made
by the oracle pass, a code moved away from a .5 boundary fails, and a code
moved within 1e-3 of one passes."""
import numpy as np
import pytest

from oracle import kv as okv
from oracle import quant as oq
from parity import check_asym, check_sym_codes


def _rows():
    # max|y| = 3.5 gives s = 0.5 exactly; u = y / s
    y = np.array([[3.5, 1.2502, -0.6, 2.0, 0.1, -3.5, 3.2495, 1.9]])
    return y, np.array([0.5], dtype=np.float16)


def test_sym_rule_accepts_the_oracle_and_near_ties():
    y, s = _rows()
    q = oq.sym_quant_with_scale(y, s)
    check_sym_codes(oq.pack_int4(q), s, y, 1.0)
    near = q.copy()
    near[0, 1] += 1          # u = 2.5004: within 1e-3 of 2.5, either neighbour is fine
    check_sym_codes(oq.pack_int4(near), s, y, 1.0)


@pytest.mark.parametrize("pos", [0, 2, 3, 4, 7])
def test_sym_rule_rejects_a_flip_away_from_a_tie(pos):
    y, s = _rows()
    q = oq.sym_quant_with_scale(y, s)
    q[0, pos] += -1 if q[0, pos] > -8 else 1
    with pytest.raises(AssertionError):
        check_sym_codes(oq.pack_int4(q), s, y, 1.0)


def test_sym_rule_rejects_a_scale_two_ulps_off():
    y, s = _rows()
    s2 = (s.view(np.uint16) + 2).view(np.float16)
    q = oq.sym_quant_with_scale(y, s2)
    with pytest.raises(AssertionError):
        check_sym_codes(oq.pack_int4(q), s2, y, 1.0)


def test_sym_rule_follows_the_stored_scale():
    # A scale one ulp below the oracle's is allowed (R2); the codes must then be
    # those of that stored scale, not of the oracle's.
    y, s = _rows()
    s1 = (s.view(np.uint16) - 1).view(np.float16)
    q1 = oq.sym_quant_with_scale(y, s1)
    check_sym_codes(oq.pack_int4(q1), s1, y, 1.0)
    q0 = oq.sym_quant_with_scale(y, s)
    assert not np.array_equal(q0, q1)
    with pytest.raises(AssertionError):
        check_sym_codes(oq.pack_int4(q0), s1, y, 1.0)


def test_asym_rule():
    rng = np.random.default_rng(7)
    y = rng.standard_normal((3, 256))
    q, s, m = okv.asym_quant_math(y, 128, 0.95)
    check_asym(q, s, m, y, 128, 0.95)
    tie = okv.asym_tie_distance(y, 128, s, m)
    far = np.argwhere(tie > 0.1)[0]
    bad = q.copy()
    bad[tuple(far)] = bad[tuple(far)] + 1 if bad[tuple(far)] < 15 else bad[tuple(far)] - 1
    with pytest.raises(AssertionError):
        check_asym(bad, s, m, y, 128, 0.95)
