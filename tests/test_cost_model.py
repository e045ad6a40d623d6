"""The per-phase cost model against phase times measured on MI355X.

The committed samples were measured by sparse_mixture_experts_route_amd.cost_model
(its main()) on one MI355X. The model is fitted on the fitting shapes only and
must predict the held-out shapes (other E, k, d_model, d_expert, including E not
a multiple of 64 and a 256-expert layer outside the fitting range) within a mean
absolute percentage error of 15 %, per phase, for the whole layer and for its
MFU (the yardstick of the MOSAIC summary's operator-level performance model,
"Compute-Optimal Is Not Cluster-Optimal", method item 2).
"""

import pytest

from sparse_mixture_experts_route_amd import cost_model as cm


@pytest.fixture(scope="module")
def samples():
    s = cm.load_samples(cm.SAMPLES_FILE)
    assert [(x.T, x.d_model, x.E, x.k, x.d_expert) for x in s] == cm.FIT_SHAPES + cm.HELD_OUT_SHAPES
    return s


def test_held_out_mape_below_15_percent(samples):
    n = len(cm.FIT_SHAPES)
    model = cm.fit(samples[:n])
    err = cm.mape(model, samples[n:])
    assert all(err[p] < 15.0 for p in cm.PHASES + ("step", "mfu")), err


def test_samples_are_consistent(samples):
    for s in samples:
        assert sum(s.counts) == s.T * s.k and len(s.counts) == s.E
        assert all(s.phases_us[p] > 0 for p in cm.PHASES)


def test_tile_choice_and_split_rule():
    # the 8-wave 256 x 256 tile for the Mixtral-shaped layer; small layers take
    # smaller tiles to fill the CUs
    assert cm.SHAPES[cm.pick_tile(8192, 2048, 8192, 8)][0] == "256x256w8"
    assert cm.SHAPES[cm.pick_tile(2048, 2048, 8192, 8)][0] == "128x128"
    # a leftover round is split only when small and K is long
    assert cm._split(10, 32, 128) and not cm._split(11, 32, 128) and not cm._split(10, 32, 16)
    assert not cm._split(0, 32, 128)


def test_prediction_scales_with_work():
    m = cm.calibrated()
    a = m.predict(4096, 2048, 8, 2, 8192)
    b = m.predict(8192, 2048, 8, 2, 8192)
    assert b["ffn"] > 1.6 * a["ffn"] and b["step"] > a["step"]
    assert set(a) == set(cm.PHASES) | {"step"}
