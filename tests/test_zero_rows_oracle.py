"""The zero-weight test matrices (tests/zero_rows.py) hold exactly the zero
weights they claim, according to the oracle's decoder (itself pinned by the
golden blocks and the independent encoder): the parity cases that use them
then really test cancellation."""
import numpy as np
import pytest

import oracle
import zero_rows as Z

TYPES = [Z.Q4_0, Z.Q8_0, Z.Q4_K, Z.Q6_K, Z.Q5_0, Z.Q5_K]


@pytest.mark.parametrize("t", TYPES)
def test_zero_row_kinds(t):
    be = Z.PK.BE[t]
    n, k = 5, 2 * be
    w = Z.make_matrix(t, n, k, ["zero", "sparse", "single", "dense", "random"], np.random.default_rng(t))
    W = oracle.dequant(t, w, n, k)
    assert not W[0].any()                                    # all zero
    assert 1 <= np.count_nonzero(W[1]) <= 2 * (k // be)      # two per block at most
    assert np.count_nonzero(W[2]) <= 1                       # one in the row
    assert not W[3][5::be].any()                             # the fixed zero position of every block
    assert np.count_nonzero(W[3]) >= k - 2 * (k // be)
    if t in (Z.Q4_K, Z.Q5_K):
        # the cancelling terms are large: d sc q0 alone is far from zero
        assert np.count_nonzero(W[4]) > k // 2


@pytest.mark.parametrize("t", [Z.Q4_K, Z.Q5_K])
def test_k_quant_zero_pairs_are_not_trivial(t):
    """The zero weights of the K-quant cases come from d sc q0 = dmin m with
    nonzero terms (not from d = 0 or sc = 0), and include codes that are not
    powers of two."""
    pairs = Z.PAIRS_4 if t == Z.Q4_K else Z.PAIRS_5
    assert all(s > 0 and q0 > 0 and s * q0 <= 63 for s, q0 in pairs)
    assert any(q0 & (q0 - 1) for _, q0 in pairs)
    assert max(q0 for _, q0 in pairs) <= Z.CODE_MAX[t]
