"""CPU checks of the GPU tests' natural-run code comparison (tests/harness.py): it accepts the
oracle's own codes, accepts a code one away only at a rounding point within the fp32
accumulation bound, and rejects a code one away elsewhere (mistakes planted on the CPU)."""

import dataclasses
import types

import numpy as np

from oracle import starkv_oracle as O
from rank_kv_cache_starkv_amd import inputs as I
from tests import harness as H


def _tiny_run():
    w = dataclasses.replace(I.WORKLOADS[2], H_q=2, H_kv=2, d_h=32, d=64, key_ranks=(9, 6), r_v=12, B=1)
    lf = I.layer_factors(w)
    OL = O.build_layer(lf.U_k, lf.s_k, lf.V_k, lf.tau_k, lf.U_v, lf.s_v, lf.V_v, lf.tau_v, w.H_q, w.latent, w.dtype)
    Xc = I.as_dtype(I.x_calibration(w), w.dtype)
    sc = O.calibrate_scales(Xc, OL.A_cat, O.channel_qmax(OL))
    X = I.as_dtype(I.x_prefill(w, 0, 0, 40), w.dtype)
    oc = O.compress(X, OL, sc)
    return types.SimpleNamespace(OL=OL, scales_o=sc, xs={0: X}, ocache={0: oc},
                                 scale_diff=np.zeros(sc.shape, bool)), X


def test_natural_code_check_accepts_the_oracle_codes():
    run, _ = _tiny_run()
    assert H.check_natural_codes(run, 0, run.ocache[0].key.copy(), run.ocache[0].value.copy()) == 0


def test_natural_code_check_rejects_a_code_off_by_one_away_from_rounding_points():
    run, X = _tiny_run()
    y = O.latent(X, run.OL.A_cat) / np.asarray(run.scales_o, np.float16).astype(np.float32)
    dist = np.abs(np.abs(y) - (np.floor(np.abs(y)) + 0.5))
    qm = O.channel_qmax(run.OL)
    ok = (dist > 0.1) & (np.abs(y) < qm - 1)
    t, c = map(int, np.argwhere(ok)[0])
    gk, gv = run.ocache[0].key.copy(), run.ocache[0].value.copy()
    nk = gk.shape[1]
    if c < nk:
        gk[t, c] += 1
    else:
        gv[t, c - nk] += 1
    try:
        H.check_natural_codes(run, 0, gk, gv)
    except AssertionError:
        return
    raise AssertionError("a planted code error passed the check")


def test_natural_code_check_accepts_one_off_at_a_rounding_point():
    run, X = _tiny_run()
    A = run.OL.A_cat
    sc = np.asarray(run.scales_o, np.float16).astype(np.float32)
    # move one token's latent onto a half-integer multiple of its channel's scale: x = 2.5 s
    c = 1
    x = O.latent(X, A)
    t = 3
    target = np.float64(2.5) * np.float64(sc[c])
    # solve for a hidden-state change along the channel's column of A that lands x exactly there
    a = A[:, c].astype(np.float64)
    X2 = X.astype(np.float64).copy()
    X2[t] += (target - float(x[t, c])) * a / float(a @ a)
    run.xs[0] = X2
    oc = O.compress(X2, run.OL, run.scales_o)
    run.ocache[0] = oc
    y = float(O.latent(X2, A)[t, c]) / float(sc[c])
    assert abs(abs(y) - 2.5) < 1e-5
    gk, gv = oc.key.copy(), oc.value.copy()
    gk[t, c] = 3 if oc.key[t, c] == 2 else 2  # the other side of the tie
    assert H.check_natural_codes(run, 0, gk, gv) == 1
