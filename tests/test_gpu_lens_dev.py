"""GPU parity of the device-length form of the hot calls: lens_host is an upper bound that sizes
the plan, and the kernels take each sequence's length from lens_dev when they run.

- decode_attention (and the hidden-state form) with bounds past the lengths, over caches whose
  bytes past each length are poisoned (0xFF: NaN for bf16 and fp32 latents), against the oracle
  at the true lengths;
- compress_append with a bound: the same cache bytes as the append at the host lengths;
- a decode step captured once in a HIP graph at capacity bounds and replayed while the graph
  itself advances lens_dev: every replay's output against the oracle and its cache bytes against
  the oracle's (exact-latent conditioning, so the codes are the oracle's bit for bit);
- rotary layers that attend over reconstructed keys refuse lens_dev.

Bars: as the other parity tests (fp32 max|err| <= 1e-4; bf16 workloads normwise 2e-2 per
(row, head)); cache bytes bit-exact."""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import starkv_oracle as O
from rank_kv_cache_starkv_amd import inputs as I

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import harness as H  # noqa: E402
else:  # collected on CPU-only machines but never run there (marked gpu)
    H = None

MINI = {0: [256], 1: [300, 129], 2: [250, 70], 3: [1000], 4: [100, 33, 257], 5: [250, 70], 6: [250, 70]}


def _setup(cfg, lens0, headroom, exact=False, n_q=None):
    w = dataclasses.replace(I.WORKLOADS[cfg], B=len(lens0))
    if n_q is not None:
        w = dataclasses.replace(w, n_q=n_q)
    run = H.make_layer(w, exact=exact)
    H.calibrate(run)
    T_max = -(-(max(lens0) + max(w.n_append, 1) + headroom) // 32) * 32
    H.prefill(run, lens0, oracle_seqs=range(len(lens0)), T_max=T_max)
    if w.n_append:
        H.append_step(run, w.n_append)
    return w, run


def _poison_tail(run, b: int, T: int) -> None:
    """Bytes 0xFF in sequence b's key rows from position T on and in its value tiles past the
    tile that holds position T - 1 (whole tiles: the packed layouts keep several tokens in one
    byte)."""
    c = run.cache
    fmt = run.fmt
    kb = c.k_rows.numel() // c.B
    k = c.k_rows[b * kb:(b + 1) * kb].view(c.T_max, fmt.k_row_bytes)
    k[T:] = 0xFF
    vb = c.v_tiles.numel() // c.B
    v = c.v_tiles[b * vb:(b + 1) * vb].view(fmt.v_rows // 32, c.T_max // O.TT, -1)
    v[:, -(-T // O.TT):] = 0xFF


def _bounds(run, extra) -> np.ndarray:
    """Upper bounds lens + extra[b], capped at the capacity."""
    return np.minimum(run.lens + np.asarray(extra[: len(run.lens)], np.int32), run.cache.T_max).astype(np.int32)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6])
def test_decode_with_device_lengths(cfg):
    """Bounds 0 .. 300 tokens past the lengths (so whole chunks and splits past a length, and for
    the longer bounds a different split plan) give the oracle's output at the true lengths."""
    w, run = _setup(cfg, MINI[cfg], headroom=320)
    bound = _bounds(run, [290, 0, 77])
    for b in range(len(run.lens)):
        _poison_tail(run, b, int(run.lens[b]))
    torch.cuda.synchronize()
    H.log(f"[lens_dev decode] cfg={cfg} {w.name} lens={run.lens.tolist()} bounds={bound.tolist()}")
    q = H.queries(run)
    lens_dev = torch.tensor(run.lens, dtype=torch.int32, device=H.DEV)
    out = run.GL.decode(run.cache, H.to_dev(q, w.dtype), bound, lens_dev=lens_dev)
    torch.cuda.synchronize()
    got = H.from_dev(out)
    for b in run.oracle_seqs:
        H.check_output(w, got[b], H.oracle_decode(run, q, b), f"len {int(run.lens[b])} bound {int(bound[b])}")
    # lens_dev at the bounds themselves reads the poisoned tokens: the host-length form must not
    # be what ran above (a NaN or a different output shows it); checked on the bf16/fp32 latents
    if w.latent in ("bf16", "f32") and int(np.max(bound - run.lens)) > 0:
        lens_dev.copy_(torch.from_numpy(bound))
        bad = H.from_dev(run.GL.decode(run.cache, H.to_dev(q, w.dtype), bound, lens_dev=lens_dev))
        torch.cuda.synchronize()
        b = int(np.argmax(bound - run.lens))
        assert not np.array_equal(bad[b], got[b])


def test_decode_hidden_with_device_lengths():
    """The hidden-state query form (absorbed W_q B_g^T) with device lengths."""
    w, run = _setup(1, MINI[1], headroom=320)
    bound = _bounds(run, [250, 31])
    for b in range(len(run.lens)):
        _poison_tail(run, b, int(run.lens[b]))
    W = I.as_dtype(I.query_weights(w), w.dtype)
    run.GL.absorb_query(H.to_dev(W, w.dtype))
    x = I.as_dtype(I.query_hidden(w), w.dtype)
    lens_dev = torch.tensor(run.lens, dtype=torch.int32, device=H.DEV)
    out = run.GL.decode_hidden(run.cache, H.to_dev(x, w.dtype), bound, lens_dev=lens_dev)
    torch.cuda.synchronize()
    got = H.from_dev(out)
    for b in run.oracle_seqs:
        ref = O.decode(O.query_from_hidden(x[b], W, w.H_q, w.d_h), run.ocache[b], run.OL, w.n_q, run.scales_o)
        H.check_output(w, got[b], ref, f"hidden len {int(run.lens[b])} bound {int(bound[b])}")


@pytest.mark.parametrize("cfg", [1, 2, 4, 6])
def test_append_with_device_lengths(cfg):
    """compress_append with lens_dev and a bound writes the bytes of the append at the host
    lengths (the same kernels, positions taken on the device)."""
    w, run = _setup(cfg, MINI[cfg], headroom=200)
    n_new = 5
    lens_pre = run.lens.copy()
    bound = np.minimum(lens_pre + 150, run.cache.T_max - n_new).astype(np.int32)
    Xn = H.to_dev(H.hidden(run, I.x_new(w, n_new, step=7)), w.dtype)
    k0, v0 = run.cache.k_rows.clone(), run.cache.v_tiles.clone()
    run.GL.append(run.cache, Xn, lens_pre)
    torch.cuda.synchronize()
    ka, va = run.cache.k_rows.clone(), run.cache.v_tiles.clone()
    run.cache.k_rows.copy_(k0)
    run.cache.v_tiles.copy_(v0)
    run.GL.append(run.cache, Xn, bound, lens_dev=torch.tensor(lens_pre, dtype=torch.int32, device=H.DEV))
    torch.cuda.synchronize()
    H.log(f"[lens_dev append] cfg={cfg} lens={lens_pre.tolist()} bounds={bound.tolist()} n_new={n_new}")
    assert torch.equal(run.cache.k_rows, ka), "key rows"
    assert torch.equal(run.cache.v_tiles, va), "value tiles"


@pytest.mark.parametrize("cfg,lens0,rope", [(0, [256], None), (1, [300, 129], None), (2, [250, 70], None),
                                            (4, [100, 33, 257], None), (6, [250, 70], None),
                                            (1, [300, 129], 10000.0), (4, [100, 33, 257], 10000.0)])
def test_graph_replay_advances_device_lengths(cfg, lens0, rope):
    """One decode step captured in a HIP graph with lens_host at the capacity and the graph's own
    lens_dev += n_q after the step; three replays append and attend at growing lengths."""
    n_steps = 3
    w, run = _setup(cfg, lens0, headroom=n_steps * 8 + 64, exact=True)
    if rope:
        run.GL.set_rope(rope)
    B, n_q = len(lens0), w.n_q
    cap = np.full(B, run.cache.T_max, np.int32)
    H.log(f"[lens_dev graph] cfg={cfg} {w.name} lens={run.lens.tolist()} capacity={run.cache.T_max} n_q={n_q} "
          f"rope={rope}")
    for b in range(B):
        _poison_tail(run, b, int(run.lens[b]))
    lens_dev = torch.tensor(run.lens + n_q, dtype=torch.int32, device=H.DEV)
    X_buf = torch.zeros((B, n_q, w.d), dtype=run.GL.torch_dtype, device=H.DEV)
    q_buf = torch.zeros((B, n_q, w.H_q, w.d_h), dtype=run.GL.torch_dtype, device=H.DEV)
    out = torch.empty_like(q_buf)
    ws = torch.empty((run.GL.workspace_bytes(B, n_q, cap),), dtype=torch.uint8, device=H.DEV)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run.GL.step(run.cache, X_buf, q_buf, cap, out=out, ws=ws, lens_dev=lens_dev)
            lens_dev.add_(n_q)
    torch.cuda.synchronize()
    for i in range(n_steps):
        Xn = H.hidden(run, I.x_new(w, n_q, step=20 + i))
        run.lens = run.lens + n_q
        q = H.queries(run, step=20 + i)
        X_buf.copy_(H.to_dev(Xn, w.dtype))
        q_buf.copy_(H.to_dev(q, w.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = H.from_dev(out)
        for b in range(B):
            H.extend_oracle(run, b, Xn[b])
        H.compare_cache(run, exact=True)
        for b in range(B):
            if rope:
                ref = O.decode(q[b].astype(np.float64), run.ocache[b], run.OL, n_q, run.scales_o, rope_theta=rope,
                               rotary_dim=w.d_h)
            else:
                ref = H.oracle_decode(run, q, b, mode="latent")
            H.check_output(w, got[b], ref, f"replay {i} seq {b} len {int(run.lens[b])}")
    assert torch.equal(lens_dev.cpu(), torch.from_numpy(run.lens + n_q)), "lens_dev advanced by the graph"
    del graph


def test_reconstruction_decode_refuses_device_lengths():
    """A rotary layer with more than 32 query rows per KV head (8 query heads per KV head x 5
    queries) attends over reconstructed keys, planned on host lengths only: lens_dev is refused
    with EUNSUPPORTED before any launch, and the same layer with 4 queries (32 rows) takes it."""
    from rank_kv_cache_starkv_amd import StarKVError
    w = dataclasses.replace(I.WORKLOADS[1], B=1, H_q=16, H_kv=2, d_h=64, d=1024, n_q=5, r_v=128, rank_lo=16,
                            rank_hi=48, rank_sum=64)
    run = H.make_layer(w)
    run.GL.set_rope(10000.0)
    cache = run.GL.new_cache(1, 128, zero=True)
    lens_dev = torch.tensor([100], dtype=torch.int32, device=H.DEV)
    q = torch.zeros((1, 5, w.H_q, w.d_h), dtype=run.GL.torch_dtype, device=H.DEV)
    with pytest.raises(StarKVError) as ei:
        run.GL.decode(cache, q, [100], lens_dev=lens_dev)
    assert ei.value.status == -4
    out = run.GL.decode(cache, q[:, :4].contiguous(), [100], lens_dev=lens_dev)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
