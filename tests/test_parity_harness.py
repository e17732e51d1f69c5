"""CPU tests of the parity harness: it accepts a result that differs from the
oracle only by an alternative decision at a near-boundary position, and
rejects one with a planted arithmetic error."""
import numpy as np
import pytest

import parity
from oracle import oracle as ORC
from quantized_softmax_attention_kia_amd.inputs import make_inputs


def _setup(calib, recon):
    q, k, v, do = make_inputs(1, 1, 300, 64, 5, q_scale=4.0)
    cfg = ORC.OracleConfig(calib, recon, "prob", "full", 16, 8.0)
    return cfg, q[0, 0], k[0, 0], v[0, 0], do[0, 0]


@pytest.mark.parametrize("calib,recon", [("fwm", "nearest"), ("minmax", "lerp"), ("minmax", "nearest")])
def test_accepts_alternative_decision(calib, recon):
    cfg, q, k, v, do = _setup(calib, recon)
    guard = 1e-3                      # wide, so that this small case has flagged positions
    ref = ORC.head(cfg, q, k, v, do, guard=guard, flag_cap=100000)
    flags = parity.relevant_flags(ref, cfg)
    assert flags.shape[0] > 0
    tested = 0
    for f in flags[::-1]:
        flip = tuple(int(x) for x in f)
        alt = ORC.head(cfg, q, k, v, do, flips=np.array([flip]))
        got = {key: alt[key] for key in parity.KEYS}
        if not any(parity.bad_mask(got[key], ref[key]).any() for key in parity.KEYS):
            continue                  # this flip stays within tolerance: nothing to explain
        rep = parity.check_head(cfg, q, k, v, do, got, guard=guard)
        assert rep["bad0"] > 0 and len(rep["flips"]) >= 1
        tested += 1
        if tested == 2:
            break
    assert tested >= 1


@pytest.mark.parametrize("mutation", ["drop_rho_delta", "x_index", "dv_with_pl", "no_tie_split"])
def test_rejects_planted_error(mutation):
    cfg, q, k, v, do = _setup("minmax", "nearest")
    k = k.copy()
    k[7] = k[3]                       # ties, so that the tie mutation shows
    wrong = ORC.head(ORC.OracleConfig(cfg.calib, cfg.recon, cfg.ste, cfg.grad, cfg.K, cfg.tau, mutation),
                     q, k, v, do)
    got = {key: wrong[key] for key in parity.KEYS}
    with pytest.raises(AssertionError):
        parity.check_head(cfg, q, k, v, do, got)
