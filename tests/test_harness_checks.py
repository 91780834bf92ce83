"""The parity harness's own checks, on the CPU: a near-tie selection row is accepted
only if it is a valid top-16 of the oracle's scores within the tie band.  Mistakes
planted in otherwise valid rows must be rejected."""
import numpy as np
import pytest

from oracle import msa as OM
from tests import harness as H


def _row(seed, n=40, sign=1.0):
    rng = np.random.default_rng(seed)
    s = sign * (5.0 + rng.random(n))            # all of one sign, distinct
    return s


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_valid_rows_pass(sign):
    s = _row(1, sign=sign)
    own = 39
    sel = OM.select_blocks(s, own)
    H.check_valid_top16(sel, s, own)
    # swap the 15th-best older block for a 16th that ties with it within the band
    older = np.argsort(-s[:own], kind="stable")
    s2 = s.copy()
    s2[older[15]] = s2[older[14]] - 1e-6 * abs(s2[older[14]])
    alt = sorted([i for i in sel if i >= 0 and i != older[14]] + [int(older[15])])
    H.check_valid_top16(np.array(alt, np.int32), s2, own)
    # fewer than 16 visible blocks: everything up to own
    H.check_valid_top16(np.array(list(range(6)) + [-1] * 10, np.int32), s, 5)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_planted_mistakes_are_rejected(sign):
    s = _row(2, sign=sign)
    own = 39
    sel = [int(i) for i in OM.select_blocks(s, own)]
    older = [int(i) for i in np.argsort(-s[:own], kind="stable")]
    bad_rows = []
    # a clear winner dropped for the 17th
    bad_rows.append(sorted([i for i in sel if i != older[0]] + [older[15]]))
    # a repeated id in place of a winner
    r = sorted([i for i in sel if i != older[3]] + [older[4]])
    bad_rows.append(r)
    # the own block missing
    bad_rows.append(sorted([i for i in sel if i != own] + [older[15]]))
    # a block past the own block
    bad_rows.append(sorted([i for i in sel if i != older[14]] + [own + 1]))
    # unsorted
    bad_rows.append(list(reversed(sel)))
    for row in bad_rows:
        with pytest.raises(AssertionError):
            H.check_valid_top16(np.array(row, np.int32), s, own)
    # padding before ids
    with pytest.raises(AssertionError):
        H.check_valid_top16(np.array([-1] + list(range(5)) + [-1] * 10, np.int32), s, 4)


def test_negative_threshold_band_widens():
    """With negative scores the band is built from |thr|, so a choice within it passes
    (a relative factor applied to thr itself would narrow the band instead)."""
    s = -10.0 - np.arange(40) * 0.5
    own = 39
    sel = [int(i) for i in OM.select_blocks(s, own)]        # blocks 0..14 and own
    s2 = s.copy()
    s2[15] = s2[14] - 1.5e-5 * abs(s2[14])                   # inside the band
    alt = sorted([i for i in sel if i != 14] + [15])
    H.check_valid_top16(np.array(alt, np.int32), s2, own)
