"""The CPU oracle against its pins (page values, closed forms, invariants, library evaluations)."""
import numpy as np
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_blocked_recurrence_matches_page_steps():
    """The page's streaming update on its worked example: the first block's alpha is 0 (page),
    and the second block rescales by exp(m_old - m_new) = exp(2 - 3)."""
    ex = oracle_pins.load_worked_example()
    _, _, alphas = oracle_pins.online_blocked(ex["scores"], ex["values"], int(ex["block_n"][0]))
    assert alphas[0] == 0.0
    assert alphas[1] == pytest.approx(np.exp(-1.0), rel=1e-15)


def test_empty_and_bad_arguments(orc):
    z = np.zeros((0, 1, 4, 8))
    o, lse = orc.attention(z, z, z, True, 0.5)
    assert o.shape == (0, 1, 4, 8) and lse.shape == (0, 1, 4)
    z = np.zeros((1, 1, 0, 8))
    o, lse = orc.attention(z, z, z, False, 0.5)
    assert o.shape == (1, 1, 0, 8)
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        orc.attention_rows(q, q, q, False, 1.0, [4])
    with pytest.raises(ValueError):
        orc.attention_rows(q, q, q, False, 1.0, [-1])


def test_threads_reported(orc):
    assert orc.num_threads() >= 1
