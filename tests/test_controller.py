"""Host policy of the width controller (GPU-Resident Speculative Decoding for
In-Browser LLM Inference with WebGPU, Feedback Control of Speculation Width),
checked against values computed here from the stated rules."""
import math

import pytest

from speculative_verification_amd.controller import WidthController, prior_drafts, window_size

CHEAP = {1: 1000.0, 2: 1020.0, 4: 1080.0, 8: 1150.0, 16: 1700.0}    # MI355X-like step costs (us)
DEAR = {1: 1000.0, 2: 1800.0, 4: 2500.0, 8: 3500.0, 16: 6000.0}    # wide steps expensive


def test_prior_is_a_geometric_chain():
    assert prior_drafts(1, 0.5) == 0
    assert prior_drafts(4, 0.5) == pytest.approx(0.5 + 0.25 + 0.125)
    assert prior_drafts(16, 0.5) == pytest.approx(sum(0.5 ** d for d in range(1, 9)))   # depth capped at 8
    a, D = 0.6, 7
    assert 1 + prior_drafts(8, a) == pytest.approx((1 - a ** (D + 1)) / (1 - a))        # break-even form


def test_first_width_follows_costs():
    # expected tokens per us under the prior (a = 0.5): 1/1000, 1.5/1020, 1.875/1080, 1.992/1150, 1.996/1700
    assert WidthController(CHEAP).width == 4
    ctl = WidthController(DEAR)
    assert ctl.width == 1                      # expensive device: opens with plain decoding
    assert ctl.probe == 2 and ctl.spacing == math.ceil((1800 / 1000 - 1) / 0.05)   # 16 windows
    assert WidthController(CHEAP).spacing == math.ceil((1080 / 1000 - 1) / 0.05)     # probe width 4: 2 windows


def test_acceptance_statistics_drive_the_width():
    ctl = WidthController(CHEAP)
    for _ in range(8):                          # long matches, every draft accepted at width 8
        ctl.update([(7, 8, 8)] * 16, 8)
    assert ctl.next() == 8 and ctl.expected_tokens(8) == pytest.approx(8.0)
    for _ in range(40):                         # drafts stop matching at every width
        for w in (2, 4, 8, 16):
            ctl.update([(0, 1, w)] * 16, w)
    assert ctl.next() == 1


def test_probes_after_plain_decoding():
    ctl = WidthController(DEAR)
    seq = [ctl.next() for _ in range(40)]
    assert seq[:15] == [1] * 15 and seq[15] == 2 and seq[16:31] == [1] * 15 and seq[31] == 2


def test_cost_ema_from_window_intervals():
    ctl = WidthController(CHEAP, ema=0.25)
    ctl.update([(1, 2, 4)] * 8, 4, window_us=8 * 2000.0)
    assert ctl.cost[4] == pytest.approx(1080 + 0.25 * (2000 - 1080))
    before = dict(ctl.cost)
    ctl.update([(1, 2, 4)] * 7 + [(-1, 0, 4)], 4, window_us=99999.0)   # a window with no-op steps is not a sample
    assert ctl.cost == before


def test_ema_of_accepted_counts():
    ctl = WidthController(CHEAP, ema=0.25)
    ctl.update([(4, 3, 8)], 8)
    assert ctl.acc[(3, 8)][0] == 4.0
    ctl.update([(0, 3, 8)], 8)
    assert ctl.acc[(3, 8)][0] == pytest.approx(4 + 0.25 * (0 - 4))


def test_acceptance_rate_with_censored_chains():
    ctl = WidthController(CHEAP, ema=0.25, prior_accept=0.5)
    assert ctl.rate(5) == pytest.approx(0.5)
    ctl.update([(3, 5, 4), (1, 5, 4)], 4)        # depth 3: one chain cut by the depth, one rejected after 1
    assert (ctl.succ[5], ctl.fail[5]) == (4.0, 1.0)
    assert ctl.rate(5) == pytest.approx((4 + 1) / (4 + 1 + 2))
    ctl.update([], 4)                             # a window decays the counts
    assert (ctl.succ[5], ctl.fail[5]) == (3.0, 0.75)
    ctl.update([(0, 5, 1)], 1)                    # width 1 has no drafts: no evidence
    assert ctl.succ[5] == pytest.approx(2.25) and ctl.fail[5] == pytest.approx(0.5625)


def test_saturated_width_pulls_wider():
    """Every draft accepted at width 4: the observed rate, not the fixed
    prior, estimates width 8, which then wins on tokens per microsecond."""
    ctl = WidthController(CHEAP)
    assert ctl.width == 4
    for _ in range(4):
        ctl.update([(3, 8, 4)] * 16, 4)
    assert ctl.rate(8) > 0.95
    assert ctl.next() == 8
    for _ in range(4):
        ctl.update([(7, 8, 8)] * 16, 8)
    assert ctl.next() == 8                        # 16 costs more than its ninth token is worth


def test_stale_statistics_fall_back_to_the_rate():
    ctl = WidthController(CHEAP, stale=2)
    ctl.update([(0, 8, 8)] * 16, 8)               # width 8 rejected everything once
    assert ctl._est(8, 8) == 0.0
    for _ in range(3):
        ctl.update([(3, 8, 4)] * 16, 4)           # since then width 4 accepts everything
    assert ctl._est(8, 8) == pytest.approx(prior_drafts(8, ctl.rate(8)))


def test_window_size_rule():
    assert window_size({1: 100.0, 2: 92.0, 4: 90.0}) == 2      # 92 <= 1.1 * 90
    assert window_size({1: 130.0, 2: 120.0, 4: 100.0}) == 4
    assert window_size({1: 99.0, 2: 95.0, 4: 90.0}) == 1
