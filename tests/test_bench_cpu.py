"""CPU checks of bench.py's roofline arithmetic: the algorithmic flops of the decode contractions
against a count written out on a tiny shape, and the choice of the binding bound (the larger of
the HBM and MFMA ideal times)."""

import dataclasses

import numpy as np
import pytest

import bench
from rank_kv_cache_starkv_amd import inputs as I


def _tiny():
    return dataclasses.replace(I.WORKLOADS[2], H_q=4, H_kv=2, d_h=8, d=32, B=2, n_q=3)


def test_decode_flops_counted():
    """Key scores: every query row (n_q queries x H_q heads) against its KV head's r_g channels of
    every cached token; values: every row against the r_v channels; up-projection: r_v x d_h per
    row, head and query.  Counted by explicit loops on a tiny GQA shape."""
    w = _tiny()
    ranks, r_v = [3, 5], 7
    lens = np.array([10, 4])
    G = w.H_q // w.H_kv
    sc = va = up = 0
    for b in range(w.B):
        for j in range(w.n_q):
            for h in range(w.H_q):
                g = h // G
                for _t in range(int(lens[b])):
                    sc += 2 * ranks[g]
                    va += 2 * r_v
                up += 2 * r_v * w.d_h
    fl = bench.algorithmic_flops(w, ranks, r_v, lens, w.n_q)
    assert fl["decode_scores"] == (float(sc), "i8")
    assert fl["decode_values"] == (float(va), "f16")
    assert fl["decode_upproj"] == (float(up), "bf16")


@pytest.mark.parametrize("byts,flops,us,bound", [
    (248.3e6, (127.1e9, "f16"), 150.0, "mfma"),  # 13B-class values: 50.8 us of MFMA > 31.0 us of HBM
    (67.1e6, (2.1e9, "bf16"), 19.0, "hbm"),      # 7B-class bf16 values: 8.4 us of HBM > 0.84 us of MFMA
    (10.0e6, None, 5.0, "hbm"),                  # no contraction: HBM only
])
def test_roofline_bound_is_the_larger_ideal_time(byts, flops, us, bound):
    r = bench.roofline_of("k", us, byts, flops, None)
    assert r["bound"] == bound
    hbm_frac = byts / (us * 1e-6) / 8e12
    if bound == "hbm":
        assert r["unit"] == "GB/s" and abs(r["frac"] - hbm_frac) < 1e-12
    else:
        mfma_frac = flops[0] / (us * 1e-6) / (bench.MFMA_PEAK[flops[1]] * 1e12)
        assert r["unit"] == "TFLOP/s" and abs(r["frac"] - mfma_frac) < 1e-12
        assert abs(r["hbm"]["frac"] - hbm_frac) < 1e-12 and abs(r["mfma"]["frac"] - mfma_frac) < 1e-12
    # the binding bound has the larger ideal time, so its fraction is the larger one
    if flops is not None:
        assert r["frac"] == max(r["hbm"]["frac"], r["mfma"]["frac"])
