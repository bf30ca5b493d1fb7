"""starkv_decode_step_noalloc (the library's static device scratch instead of a caller
workspace) against starkv_decode_step, called through the C ABI: the same output and cache bytes
bit for bit on two calls in a row, the second with a smaller input, and EWORKSPACE for a step
that needs more scratch than the library holds."""

import dataclasses

import numpy as np
import pytest
import torch

from rank_kv_cache_starkv_amd import inputs as I

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import harness as H  # noqa: E402
else:  # collected on CPU-only machines but never run there (marked gpu)
    H = None


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _case(run, w, lens0, step, slack=0):
    """The step on B = len(lens0) sequences of the run's cache: existing entry point (caller
    workspace) from a copy of the cache, then the no-alloc one from the same starting bytes.
    slack > 0: both calls take the lengths on the device, planned at lens + slack (capped at the
    cache capacity)."""
    B, n_q = len(lens0), w.n_q
    wb = dataclasses.replace(w, B=B)
    lens = np.asarray(lens0, np.int32) + n_q
    lens_dev = None
    if slack:
        lens_dev = torch.from_numpy(lens.copy()).to(H.DEV)
        lens = np.minimum(lens + slack, run.cache.T_max).astype(np.int32)
    Xn = H.to_dev(H.hidden(run, I.x_new(wb, n_q, step=step)), w.dtype)
    q = H.to_dev(I.as_dtype(I.queries(wb, step=step), w.dtype), w.dtype)
    k0, v0 = run.cache.k_rows.clone(), run.cache.v_tiles.clone()
    ws = torch.empty((run.GL.workspace_bytes(B, n_q, lens),), dtype=torch.uint8, device=H.DEV)
    ref = run.GL.step(run.cache, Xn, q, lens, out=torch.empty_like(q), ws=ws, lens_dev=lens_dev)
    torch.cuda.synchronize()
    k_ref, v_ref = run.cache.k_rows.clone(), run.cache.v_tiles.clone()
    run.cache.k_rows.copy_(k0)
    run.cache.v_tiles.copy_(v0)
    out = torch.full_like(q, float("nan"))
    run.GL.step_noalloc(run.cache, Xn, q, lens, out, lens_dev=lens_dev)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref)), "output bits"
    assert torch.equal(run.cache.k_rows, k_ref) and torch.equal(run.cache.v_tiles, v_ref), "cache bytes"
    return ref


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_noalloc_step_matches_workspace_step(cfg):
    w = I.WORKLOADS[cfg]
    lens0 = {1: [300, 129, 77], 2: [250, 70, 180], 4: [100, 33, 257, 64, 90]}[cfg]
    w = dataclasses.replace(w, B=len(lens0))
    H.log(f"[noalloc] cfg={cfg} {w.name} lens0={lens0}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=[0], T_max=max(lens0) + 2 * w.n_q + 32)
    # first call: every sequence; second call: a smaller input (fewer, shorter sequences), which
    # finds the first call's contents in the scratch
    out1 = _case(run, w, lens0, step=1)
    sub = [min(x, 40) for x in lens0[:2]]
    out2 = _case(run, w, sub, step=2)
    assert out1.shape[0] == len(lens0) and out2.shape[0] == 2
    # the oracle's bar for the first sequence of the first call is covered by the workspace
    # step's own parity tests; the two entry points agree bit for bit


def test_noalloc_step_with_device_lengths():
    """The no-alloc step with lengths on the device (planned 200 tokens past them) against the
    workspace step with the same arguments, bit for bit, on two calls in a row."""
    w = I.WORKLOADS[2]
    lens0 = [250, 70, 180]
    w = dataclasses.replace(w, B=len(lens0))
    H.log(f"[noalloc lens_dev] cfg=2 lens0={lens0}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=[0], T_max=max(lens0) + 2 * w.n_q + 256)
    _case(run, w, lens0, step=3, slack=200)
    _case(run, w, [min(x, 40) for x in lens0[:2]], step=4, slack=100)


def test_noalloc_refuses_a_step_beyond_its_scratch():
    """The full 13B-class ragged step needs more workspace than the static scratch: EWORKSPACE,
    with nothing enqueued."""
    import rank_kv_cache_starkv_amd as S
    w = I.WORKLOADS[4]
    lens = (I.context_lengths(w) + w.n_q).astype(np.int32)
    lf = I.layer_factors(w)
    GL = S.Layer(w.H_q, w.H_kv, w.d_h, w.d, w.dtype, w.latent, lf.s_k, lf.tau_k, lf.s_v, lf.tau_v)
    dev = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(H.DEV) for a in (lf.U_k, lf.V_k, lf.U_v, lf.V_v)]
    GL.build_factors(*dev)
    GL.bind_scales(torch.ones((GL.info["n_lat"],), dtype=torch.float16, device=H.DEV))
    assert GL.workspace_bytes(w.B, w.n_q, lens) > S.NOALLOC_SCRATCH_BYTES
    cache = GL.new_cache(w.B, 32 * (-(-int(lens.max()) // 32)))
    q = torch.zeros((w.B, w.n_q, w.H_q, w.d_h), dtype=torch.bfloat16, device=H.DEV)
    X = torch.zeros((w.B, w.n_q, w.d), dtype=torch.bfloat16, device=H.DEV)
    out = torch.empty_like(q)
    with pytest.raises(S.StarKVError) as ei:
        GL.step_noalloc(cache, X, q, lens, out)
    assert ei.value.status == -5
    GL.close()
