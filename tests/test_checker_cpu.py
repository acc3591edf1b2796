"""The selection checker of the GPU parity tests, on hand-made selections
(CPU).  It must accept exactly the legal selections: the sink, the current
block and top_k - 2 candidates none of which an excluded candidate beats by
more than the tie tolerance, or every block when there are at most top_k."""
import math

from tests.spla_parity import TIE_REL, check_selection


def _lg(nb, scores):
    return {j: scores[j - 1] for j in range(1, nb - 1)}


def test_accepts_the_exact_top_k():
    nb, top_k = 10, 4
    lg = _lg(nb, [0.1, 0.9, 0.3, 0.8, 0.2, 0.4, 0.0, 0.5])  # candidates 1..8
    assert check_selection([0, 2, 4, 9], lg, nb, top_k) is None


def test_rejects_a_beaten_candidate():
    nb, top_k = 10, 4
    lg = _lg(nb, [0.1, 0.9, 0.3, 0.8, 0.2, 0.4, 0.0, 0.5])
    msg = check_selection([0, 2, 3, 9], lg, nb, top_k)  # 3 (0.3) in, 4 (0.8) out
    assert msg is not None and "beaten" in msg


def test_accepts_a_swap_inside_the_tie_tolerance():
    nb, top_k = 6, 3
    x = 1.0
    lg = _lg(nb, [x, x * (1 + 0.5 * TIE_REL), 0.0, -1.0])
    # candidate 2 is larger by half the tolerance in log terms: either pick is legal
    assert check_selection([0, 1, 5], lg, nb, top_k) is None
    assert check_selection([0, 2, 5], lg, nb, top_k) is None
    lg_far = _lg(nb, [x, x - 10 * math.log1p(-TIE_REL), 0.0, -1.0])
    assert check_selection([0, 1, 5], lg_far, nb, top_k) is not None


def test_top_k_two_is_sink_and_current():
    nb = 185
    lg = _lg(nb, [float(j % 7) for j in range(1, nb - 1)])
    assert check_selection([0, nb - 1], lg, nb, 2) is None
    assert check_selection([0, 5], lg, nb, 2) is not None


def test_every_block_when_at_most_top_k():
    assert check_selection([0, 1, 2, -1, -1], {1: 0.0}, 3, 5) is None
    assert check_selection([0, 2, -1, -1, -1], {1: 0.0}, 3, 5) is not None


def test_padding_and_order():
    lg = _lg(10, [0.0] * 8)
    assert "padding" in check_selection([0, -1, 3, 9], lg, 10, 4)
    assert "ascending" in check_selection([0, 3, 2, 9], lg, 10, 4)
    assert "sink/current" in check_selection([1, 2, 3, 4], lg, 10, 4)
