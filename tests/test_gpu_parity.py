"""GPU parity: libstarkv on the MI355X against the CPU oracle (same seeded inputs).

Bars: ranks, factor bits, scales and cache bytes bit-exact (exact-latent conditioning);
decode outputs within max|err| <= 1e-4 (fp32 workload) or normwise relative 2e-2 (bf16
workloads); the same call twice gives bit-identical outputs.
"""

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


# ---------------------------------------------------------------- factors and ranks, full shapes

@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6])
def test_ranks_and_factor_bits(cfg):
    w = I.WORKLOADS[cfg]
    H.log(f"[factors] cfg={cfg} {w.name}")
    run = H.make_layer(w, exact=False)
    assert list(run.GL.ranks) == list(map(int, run.OL.ranks)), "ranks"
    assert run.GL.r_v == run.OL.r_v
    np.testing.assert_array_equal(H.dev_bits(run.GL.A_t), H.f32_bits(run.OL.A_cat.T, w.dtype))
    np.testing.assert_array_equal(H.dev_bits(run.GL.B_k), H.f32_bits(run.OL.B_k, w.dtype))
    np.testing.assert_array_equal(H.dev_bits(run.GL.B_vt), H.f32_bits(run.OL.B_v.T, w.dtype))
    fmt = run.fmt
    assert run.GL.info["k_row_bytes"] == fmt.k_row_bytes and run.GL.info["v_tile_rows"] == fmt.v_rows


# ---------------------------------------------------------------- reduced-size workloads, every element

def mini(cfg):
    w = I.WORKLOADS[cfg]
    lens = {0: [256], 1: [300, 129], 2: [250, 70], 3: [1000], 4: [100, 33, 257], 5: [250, 70], 6: [250, 70]}[cfg]
    return w, lens


def _run_mini(cfg, exact, q_scale=1.0):
    w, lens0 = mini(cfg)
    w = dataclasses.replace(w, B=len(lens0))
    H.log(f"[mini] cfg={cfg} {w.name} exact={exact} lens0={lens0} n_append={w.n_append} q_scale={q_scale}")
    run = H.make_layer(w, exact=exact)
    H.calibrate(run)  # scales: bit-exact (exact-latent), or within the accumulation bound (natural)
    H.prefill(run, lens0, oracle_seqs=range(len(lens0)))
    if w.n_append:
        H.append_step(run, w.n_append)
    return w, run


def _compare_cache(run, exact):
    H.compare_cache(run, exact)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("exact", [True, False])
def test_mini_parity(cfg, exact):
    w, run = _run_mini(cfg, exact)
    _compare_cache(run, exact)
    q = H.queries(run)
    out = H.decode(run, q)
    out2 = H.decode(run, q)
    assert torch.equal(out.view(torch.int16) if out.dtype != torch.float32 else out.view(torch.int32),
                       out2.view(torch.int16) if out2.dtype != torch.float32 else out2.view(torch.int32)), "determinism"
    got = H.from_dev(out)
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b)
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6])
def test_absorbed_query_from_hidden(cfg):
    """Decode with the query taken from hidden states through the absorbed factors W_q^h B_g^T,
    against the oracle's q = x W_q followed by the same attention (at most 16 hidden rows: the
    8-row skinny projection GEMM, and the 16-row one for the 13B-class mini's 12 rows)."""
    from rank_kv_cache_starkv_amd import StarKVError
    w, run = _run_mini(cfg, exact=True)
    B = len(run.lens)
    x = I.as_dtype(I.query_hidden(dataclasses.replace(w, B=B)), w.dtype)
    W = I.as_dtype(I.query_weights(w), w.dtype)
    xd, Wd = H.to_dev(x, w.dtype), H.to_dev(W, w.dtype)
    with pytest.raises(StarKVError) as ei:
        run.GL.decode_hidden(run.cache, xd, run.lens)
    assert ei.value.status == -7  # ESTATE: nothing absorbed yet
    run.GL.absorb_query(Wd)
    out = run.GL.decode_hidden(run.cache, xd, run.lens)
    out2 = run.GL.decode_hidden(run.cache, xd, run.lens)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "determinism"
    got = H.from_dev(out)
    for b in run.oracle_seqs:
        q = O.query_from_hidden(x[b], W, w.H_q, w.d_h)
        ref = O.decode(q, run.ocache[b], run.OL, w.n_q, run.scales_o)
        H.check_output(w, got[b], ref, f"hidden-state query seq {b} len {int(run.lens[b])}")
    # binding factors again drops the absorbed ones
    run.GL.bind_factors(run.GL.A_t, run.GL.B_k, run.GL.B_vt)
    with pytest.raises(StarKVError) as ei:
        run.GL.decode_hidden(run.cache, xd, run.lens)
    assert ei.value.status == -7


def _small_head_mix84():
    return dataclasses.replace(I.WORKLOADS[2], H_q=4, H_kv=4, d=512, key_ranks=(20, 33, 48, 27), r_v=96)


HIDDEN_FORMS = {
    # name: (workload, batch, n_q, oracle sequences); rows = batch x n_q hidden rows
    "13b-64x4-tiled8": (I.WORKLOADS[4], 64, 4, (0, 31, 63)),  # 256 rows, XCD-mapped 8-wave tiles, bf16 hi+lo
    "gqa-8x4-tiled8": (I.WORKLOADS[3], 8, 4, (0, 7)),  # 32 rows, GQA (G = 4 absorbed copies per KV head)
    "f32-8x4-tiled8": (I.WORKLOADS[0], 8, 4, (0, 5, 7)),  # 32 rows, fp32 factors
    "f32-128x9-tiled4": (I.WORKLOADS[0], 128, 9, (0, 77, 127)),  # 1152 rows: the 4-wave grid
    "bf16-128x9-tiled4": (None, 128, 9, (0, 64, 127)),  # 1152 rows, small-head int8/int4 layer, bf16 hi+lo
}


@pytest.mark.parametrize("form", list(HIDDEN_FORMS))
def test_absorbed_query_gemm_forms(form):
    """Hidden-state queries with more than 16 rows, one case per tiled form of the projection GEMM
    (8-wave XCD-mapped tiles up to 1024 rows, 4-wave tiles beyond; fp32 factors and bf16 high +
    low parts), against the oracle's q = x W_q followed by the same attention."""
    w0, B, n_q, sample = HIDDEN_FORMS[form]
    w0 = w0 if w0 is not None else _small_head_mix84()
    w = dataclasses.replace(w0, B=B, n_q=n_q)
    lens0 = [17 + (37 * b) % 150 for b in range(B)]
    H.log(f"[hidden-query form] {form}: {w.name} B={B} n_q={n_q} rows={B * n_q} lens0 {min(lens0)}..{max(lens0)}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=sample, fast_fill=True)
    H.append_step(run, max(w.n_append, n_q))
    x = I.as_dtype(I.query_hidden(w), w.dtype)
    W = I.as_dtype(I.query_weights(w), w.dtype)
    run.GL.absorb_query(H.to_dev(W, w.dtype))
    xd = H.to_dev(x, w.dtype)
    out = run.GL.decode_hidden(run.cache, xd, run.lens)
    out2 = run.GL.decode_hidden(run.cache, xd, run.lens)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "determinism"
    got = H.from_dev(out)
    assert np.all(np.isfinite(got))
    for b in sample:
        q = O.query_from_hidden(x[b], W, w.H_q, w.d_h)
        ref = O.decode(q, run.ocache[b], run.OL, n_q, run.scales_o, mode="latent")
        H.check_output(w, got[b], ref, f"{form} seq {b} len {int(run.lens[b])}")


@pytest.mark.parametrize("cfg", [0, 2, 4, 5, 6])
@pytest.mark.parametrize("q_scale", [30.0, 300.0])
def test_mini_softmax_stress(cfg, q_scale):
    w, run = _run_mini(cfg, exact=True)
    q = H.queries(run, scale=q_scale)
    got = H.from_dev(H.decode(run, q))
    for b in run.oracle_seqs:
        H.check_output(w, got[b], H.oracle_decode(run, q, b), f"q x{q_scale} seq {b}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 5, 6])
def test_reconstruct(cfg):
    w, run = _run_mini(cfg, exact=True)
    b = 0
    T = int(run.lens[b])
    t0, t1 = 3, T
    K, V = run.GL.reconstruct(run.cache, b, t0, t1)
    torch.cuda.synchronize()
    xk, xv = O.dequantized(run.ocache[b], run.OL, run.scales_o)
    Kr, Vr = O.reconstruct(xk[t0:t1], xv[t0:t1], run.OL)
    for got, ref, name in ((H.from_dev(K), Kr, "K"), (H.from_dev(V), Vr, "V")):
        err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
        H.log(f"  reconstruct {name}: normwise rel {err:.3e}")
        assert err <= (1e-5 if w.dtype == "f32" else 2 ** -8)


# ---------------------------------------------------------------- edge cases

def test_edge_lengths_and_tails():
    """Lengths equal to n_q, to one tile, just over a chunk, and a cache with no slack."""
    w = dataclasses.replace(I.WORKLOADS[4], B=5)
    lens0 = [0, 28, 60, 61, 125]  # + 4 appended: 4, 32, 64, 65, 129
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=range(5), T_max=160)
    H.append_step(run, 4)
    _compare_cache(run, True)
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in range(5):
        H.check_output(w, got[b], H.oracle_decode(run, q, b), f"len {int(run.lens[b])}")


def test_append_noop_and_capacity():
    import rank_kv_cache_starkv_amd as S
    w = dataclasses.replace(I.WORKLOADS[0], B=1)
    run = H.make_layer(w)
    H.prefill(run, [64], oracle_seqs=[0], T_max=64)
    before = run.cache.k_rows.clone()
    run.GL.append(run.cache, torch.zeros((1, 0, w.d), device=H.DEV), [64])  # n_new = 0: no-op
    torch.cuda.synchronize()
    assert torch.equal(before, run.cache.k_rows)
    with pytest.raises(S.StarKVError) as e:
        run.GL.append(run.cache, torch.zeros((1, 1, w.d), device=H.DEV), [64])
    assert e.value.status == -3
    q = torch.zeros((1, 1, w.H_q, w.d_h), device=H.DEV)
    with pytest.raises(S.StarKVError) as e:
        run.GL.decode(run.cache, q, [65])
    assert e.value.status == -3
    with pytest.raises(S.StarKVError) as e:
        run.GL.decode(run.cache, q, [64], ws=torch.empty(256, dtype=torch.uint8, device=H.DEV))
    assert e.value.status == -5


# ---------------------------------------------------------------- full-size workloads, sampled sequences

def _full(cfg):
    w = I.WORKLOADS[cfg]
    lens0 = I.context_lengths(w)
    if cfg == 4:
        order = np.argsort(lens0)
        sample = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]  # shortest, median, longest
    else:
        sample = [0] if w.B == 1 else [0, w.B - 1]
    H.log(f"[full] cfg={cfg} {w.name} B={w.B} lens0 in [{lens0.min()}, {lens0.max()}] oracle seqs {sample}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    if O.is_quantized(w.latent):
        np.testing.assert_array_equal(H.dev_bits(run.GL.scales), run.scales_o.view(np.uint16))
    H.prefill(run, lens0, oracle_seqs=sample, fast_fill=True)
    if w.n_append:
        H.append_step(run, w.n_append)
    return w, run


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6])
def test_full_size_sampled(cfg):
    w, run = _full(cfg)
    _compare_cache(run, True)
    q = H.queries(run)
    out = H.decode(run, q)
    got = H.from_dev(out)
    assert np.all(np.isfinite(got))
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b, mode="latent")
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")


# ---------------------------------------------------------------- graph capture of a decode step

def test_graph_replay_matches_eager():
    """One decode step (append + attention) captured in a HIP graph: every replay, with eager
    work and synchronisations in between, gives the eager result bit for bit."""
    w, run = _run_mini(2, exact=True)
    q = H.to_dev(H.queries(run), w.dtype)
    Xn = H.to_dev(H.hidden(run, I.x_new(dataclasses.replace(w, B=len(run.lens)), 1, step=7)), w.dtype)
    lens_pre = run.lens.copy()
    lens = lens_pre + 1
    ws = torch.empty((run.GL.workspace_bytes(len(lens), w.n_q, lens),), dtype=torch.uint8, device=H.DEV)
    out = torch.empty_like(q)
    run.GL.append(run.cache, Xn, lens_pre)
    run.GL.decode(run.cache, q, lens, out=out, ws=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run.GL.append(run.cache, Xn, lens_pre)
            run.GL.decode(run.cache, q, lens, out=out, ws=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        ws.fill_(0xAB)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        # eager work between replays
        run.GL.decode(run.cache, q, lens, out=torch.empty_like(q))
        torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [0, 1, 2, 5, 6])
@pytest.mark.parametrize("n_new", [1, 2])
def test_append_few_tokens(cfg, n_new):
    """Appends of one or two tokens per sequence (the per-step append) on top of a prefill:
    cache bytes bit-exact against the oracle (exact-latent conditioning)."""
    w = dataclasses.replace(I.WORKLOADS[cfg], B=3)
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, [40, 31, 64], oracle_seqs=range(3), T_max=128)
    H.append_step(run, n_new, step=3)
    H.append_step(run, n_new, step=4)
    _compare_cache(run, True)
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in range(3):
        H.check_output(w, got[b], H.oracle_decode(run, q, b), f"len {int(run.lens[b])}")


# ---------------------------------------------------------------- the fused decode step

@pytest.mark.parametrize("cfg,lens0", [(0, [256]), (1, [300, 129]), (2, [250, 70]), (3, [700]),
                                       (4, [100, 33, 257]), (4, [100, 33, 257, 64, 90]), (5, [250, 70]),
                                       (6, [250, 70])])
def test_decode_step_equals_append_then_decode(cfg, lens0):
    """starkv_decode_step leaves the cache bytes and gives the output of compress_append followed
    by decode_attention, bit for bit: one fused launch for up to 16 new rows (cfg 0-3, and cfg 4
    with 3 sequences x 4 queries), the two-launch path beyond (cfg 4 with 5 sequences); the
    output also meets the oracle's bar for sequence 0."""
    w = dataclasses.replace(I.WORKLOADS[cfg], B=len(lens0))
    H.log(f"[step] cfg={cfg} {w.name} lens0={lens0} n_q={w.n_q}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=[0])
    n_q = w.n_q
    lens_pre = run.lens.copy()
    k0, v0 = run.cache.k_rows.clone(), run.cache.v_tiles.clone()
    Xn_np = H.hidden(run, I.x_new(w, n_q, step=3))
    Xn = H.to_dev(Xn_np, w.dtype)
    run.lens = lens_pre + n_q
    q_np = H.queries(run, step=3)
    q = H.to_dev(q_np, w.dtype)
    # two calls
    run.GL.append(run.cache, Xn, lens_pre)
    out_a = run.GL.decode(run.cache, q, run.lens)
    torch.cuda.synchronize()
    ka, va = run.cache.k_rows.clone(), run.cache.v_tiles.clone()
    # the fused step on the same starting cache
    run.cache.k_rows.copy_(k0)
    run.cache.v_tiles.copy_(v0)
    out_b = run.GL.step(run.cache, Xn, q, run.lens)
    torch.cuda.synchronize()
    assert torch.equal(run.cache.k_rows, ka) and torch.equal(run.cache.v_tiles, va), "cache bytes"
    bits = (lambda t: t.view(torch.int32)) if out_a.dtype == torch.float32 else (lambda t: t.view(torch.int16))
    assert torch.equal(bits(out_a), bits(out_b)), "output bits"
    oc = O.compress(Xn_np[0], run.OL, run.scales_o)
    old = run.ocache[0]
    run.ocache[0] = O.SequenceCache(np.concatenate([old.key, oc.key]), np.concatenate([old.value, oc.value]))
    ref = H.oracle_decode(run, q_np, 0, mode="latent")
    H.check_output(w, H.from_dev(out_b)[0], ref, f"seq 0 len {int(run.lens[0])}")


@pytest.mark.parametrize("cfg", [4, 5])
def test_decode_step_many_rows_natural(cfg):
    """starkv_decode_step with more than 16 new rows (10 sequences x 4 queries: the tiled append,
    then the decode) on unsnapped inputs: the new tokens' codes against the oracle's (differences
    of one code, at most at rounding ties) and the output within the bf16 bar."""
    lens0 = [60, 33, 100, 75, 41, 90, 128, 64, 50, 81]
    w = dataclasses.replace(I.WORKLOADS[cfg], B=len(lens0), n_q=4)
    H.log(f"[step many rows natural] cfg={cfg} B={w.B} rows={w.B * w.n_q}")
    run = H.make_layer(w, exact=False)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=(0, 6, 9))
    lens_pre = run.lens.copy()
    Xn_np = H.hidden(run, I.x_new(w, w.n_q, step=5))
    run.lens = lens_pre + w.n_q
    q_np = H.queries(run, step=5)
    out = run.GL.step(run.cache, H.to_dev(Xn_np, w.dtype), H.to_dev(q_np, w.dtype), run.lens)
    torch.cuda.synchronize()
    got = H.from_dev(out)
    for b in run.oracle_seqs:
        H.extend_oracle(run, b, Xn_np[b])
        gk, gv = H.gpu_seq_cache(run, b)
        T = int(run.lens[b])
        kc = O.unpack_key_rows(gk, run.fmt)[T - w.n_q: T]
        vc = O.unpack_value_tiles(gv, run.fmt, T)[T - w.n_q: T]
        nd = H.check_natural_codes(run, b, kc, vc, t0=T - w.n_q)
        H.log(f"  seq {b}: new-token codes differing by one at rounding boundaries: {nd}/{kc.size + vc.size}")
        H.check_output(w, got[b], H.oracle_decode(run, q_np, b, mode="latent"), f"seq {b} len {T}")


@pytest.mark.parametrize("cfg,n_q", [(0, 9), (1, 2), (1, 3), (2, 2), (5, 2), (5, 4)])
def test_many_query_rows(cfg, n_q):
    """More than 32 query rows per sequence (n_q queries x H_q heads): the staged many-row value
    kernel (bf16, int8/int4) and the general one (fp32) against the oracle, causal within the
    chunk of n_q queries."""
    w, lens0 = mini(cfg)
    w = dataclasses.replace(w, B=len(lens0), n_q=n_q)
    H.log(f"[rows] cfg={cfg} n_q={n_q} rows={w.H_q * n_q} lens={lens0}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=range(len(lens0)))
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b)
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")


def test_many_rows_per_kv_head():
    """64 query rows per KV head (16 sequences x 4 queries, bf16 latent): the tall up-projection
    and the staged many-row value kernel against the oracle on every sequence."""
    lens0 = [40, 75, 128, 200, 33, 64, 97, 150, 45, 81, 110, 190, 36, 70, 129, 160]
    w = dataclasses.replace(I.WORKLOADS[1], B=len(lens0), n_q=4)
    H.log(f"[tall] rows per KV head {w.B * w.n_q}, lens={lens0}")
    run = H.make_layer(w, exact=True)
    H.prefill(run, lens0, oracle_seqs=range(len(lens0)))
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b, mode="latent")
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")


def test_many_rows_per_kv_head_mix84():
    """64 query rows per KV head with int8/int4 latents (16 sequences x 4 queries): the tall
    up-projection with the split merge folded in (value scales applied per channel)."""
    lens0 = [40, 75, 128, 200, 33, 64, 97, 150, 45, 81, 110, 190, 36, 70, 129, 160]
    w = dataclasses.replace(I.WORKLOADS[2], B=len(lens0), n_q=4)
    H.log(f"[tall mix84] rows per KV head {w.B * w.n_q}, lens={lens0}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=(0, 3, 11, 15))
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b, mode="latent")
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")


@pytest.mark.parametrize("cfg", [1, 4])
def test_many_sequences(cfg):
    """32 short sequences of distinct lengths (1024 or more KV-head x sequence pairs, many score
    workgroups spanning sequence boundaries) against the oracle on the first, a middle and the last
    sequence."""
    lens0 = [40 + 7 * i for i in range(32)]
    w = dataclasses.replace(I.WORKLOADS[cfg], B=len(lens0))
    H.log(f"[many sequences] cfg={cfg} B={w.B} pairs={w.B * w.H_kv}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=(0, 13, 31), fast_fill=True)
    if w.n_append:
        H.append_step(run, w.n_append)
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b, mode="latent")
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")


@pytest.mark.parametrize("cfg", [2, 4])
def test_max_batch_skewed_lengths(cfg):
    """The largest batch (128 sequences) with a skewed length mix, every 16th sequence long and
    the rest short: the longest-first XCD order of the value splits over many splits (one query
    row tile for the 7B layer, many for the 13B-class one), against the oracle on long and short
    sequences."""
    lens0 = [1900 + 13 * i if i % 16 == 0 else 33 + 5 * i for i in range(128)]
    w = dataclasses.replace(I.WORKLOADS[cfg], B=len(lens0))
    H.log(f"[max batch, skewed] cfg={cfg} B={w.B} lens {min(lens0)}..{max(lens0)}")
    run = H.make_layer(w, exact=True)
    H.calibrate(run)
    H.prefill(run, lens0, oracle_seqs=(0, 1, 64, 127), fast_fill=True)
    if w.n_append:
        H.append_step(run, w.n_append)
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b, mode="latent")
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")


def test_many_rows_many_splits():
    """64 query rows per KV head (8 sequences x 8 queries, bf16) with a sequence long enough for
    more than four value splits: the separate split merge, then the tall up-projection."""
    lens0 = [1400, 60, 130, 300, 45, 90, 220, 75]
    w = dataclasses.replace(I.WORKLOADS[1], B=len(lens0), n_q=8)
    H.log(f"[tall, many splits] rows per KV head {w.B * w.n_q}, lens={lens0}")
    run = H.make_layer(w, exact=True)
    H.prefill(run, lens0, oracle_seqs=(0, 1, 6))
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b, mode="latent")
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")


def test_fp32_many_key_tiles():
    """fp32 latent with key ranks near d_h (396 key channels: 13 K-tiles in the one column tile,
    so every score wave takes several K-tile groups) against the oracle."""
    w = dataclasses.replace(I.WORKLOADS[0], d_h=128, d=512, key_ranks=(100, 90, 110, 96), r_v=128, B=2)
    lens0 = [300, 77]
    H.log(f"[f32 K-tiles] ranks={w.key_ranks} lens={lens0}")
    run = H.make_layer(w, exact=True)
    H.prefill(run, lens0, oracle_seqs=range(len(lens0)))
    q = H.queries(run)
    got = H.from_dev(H.decode(run, q))
    for b in run.oracle_seqs:
        ref = H.oracle_decode(run, q, b)
        H.check_output(w, got[b], ref, f"seq {b} len {int(run.lens[b])}")
