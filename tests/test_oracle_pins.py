"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test ties one oracle function to something the pages or mathematics fix:
brute force on tiny inputs, crafted ties, closed forms, textbook values and
independent library routines (numpy, scipy, torch CPU).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import MLP, ACT_GELU, ACT_IDENTITY

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- refs

def test_build_refs_are_strided_rows_bitwise():
    x = _rng(1).standard_normal((77, 9)).astype(np.float32).astype(np.float64)
    for s in (1, 2, 5, 16, 77, 100):
        r = oracle.build_refs(x, s)
        assert r.shape == (-(-77 // s), 9)
        assert np.array_equal(r.view(np.uint64), x[::s].view(np.uint64))


def test_num_refs_counts_positions_multiple_of_stride():
    for T in (0, 1, 15, 16, 17, 512, 1000):
        for s in (1, 3, 16):
            assert oracle.num_refs(T, s) == sum(1 for p in range(T) if p % s == 0)


# ------------------------------------------------------------------- top-k select

def _brute_force_select(x, s, k):
    """Independent top-k: numpy distances + lexsort by (distance, ordinal)."""
    T = x.shape[0]
    refs = x[::s]
    out = {}
    for t in range(T):
        if t % s == 0:
            continue
        cand = np.arange(len(refs))[np.arange(len(refs)) * s < t]
        dist = ((x[t][None, :] - refs[cand]) ** 2).sum(axis=1)
        order = cand[np.lexsort((cand, dist))]
        row = np.full(k, -1, np.int32)
        row[:min(k, len(order))] = order[:k]
        out[t] = row
    return out


@pytest.mark.parametrize("seed", range(12))
def test_select_matches_brute_force_on_small_integers(seed):
    # small integer coordinates: every distance is exact in any summation
    # order, and exact ties are frequent, so the tie rule is exercised
    rng = _rng(100 + seed)
    T = int(rng.integers(2, 70))
    d = int(rng.integers(1, 5))
    s = int(rng.integers(2, 6))
    k = int(rng.integers(1, 6))
    x = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
    refs = oracle.build_refs(x, s)
    pos = oracle.nonref_positions(T, s)
    if len(pos) == 0:
        return
    idx = oracle.select(x[pos], pos, refs, s, k)
    ref = _brute_force_select(x, s, k)
    for row, t in zip(idx, pos):
        assert np.array_equal(row, ref[int(t)]), (t, row, ref[int(t)])


def test_select_on_float_rows_is_a_valid_ordering():
    # fp32-valued rows at head_dim 64 (the tiny workload's shape): the chosen
    # list must be sorted by distance and no excluded ref may be closer
    rng = _rng(7)
    x = rng.standard_normal((512, 64)).astype(np.float32).astype(np.float64) * 10
    s, k = 16, 4
    refs = oracle.build_refs(x, s)
    pos = oracle.nonref_positions(512, s)
    idx = oracle.select(x[pos], pos, refs, s, k)
    for row, t in zip(idx, pos):
        n_cand = -(-int(t) // s)
        dist = ((x[t] - refs[:n_cand]) ** 2).sum(axis=1)
        k_eff = min(k, n_cand)
        assert np.all(row[k_eff:] == -1)
        chosen = row[:k_eff]
        assert np.all(np.diff(dist[chosen]) >= -1e-9 * dist.max())
        rest = np.setdiff1d(np.arange(n_cand), chosen)
        if len(rest):
            assert dist[rest].min() >= dist[chosen].max() - 1e-9 * dist.max()


def test_select_duplicate_refs_prefer_lower_position():
    s, k, d = 4, 2, 3
    x = np.zeros((21, d))
    x[0] = x[8] = x[16] = [1, 2, 3]    # refs 0, 2, 4 identical
    x[4] = x[12] = [9, 9, 9]           # refs 1, 3 far away
    x[20] = [5, 5, 5]
    x[17] = [1, 2, 3]                  # equal to refs 0, 2, 4
    pos = np.array([17])
    idx = oracle.select(x[pos], pos, oracle.build_refs(x, s), s, k)
    assert idx.tolist() == [[0, 2]]


def test_select_token_equal_to_ref_takes_it_first():
    rng = _rng(3)
    x = rng.standard_normal((40, 8))
    s, k = 5, 3
    x[33] = x[25]                      # position 25 is ref 5
    pos = np.array([33])
    refs = oracle.build_refs(x, s)
    idx = oracle.select(x[pos], pos, refs, s, k)
    assert idx[0, 0] == 5
    assert oracle.sq_dist(x[33], refs[5]) == 0.0


def test_select_short_prefix_uses_sentinels():
    rng = _rng(4)
    x = rng.standard_normal((40, 4))
    s, k = 8, 4
    refs = oracle.build_refs(x, s)
    for t, k_eff in ((1, 1), (7, 1), (9, 2), (17, 3), (25, 4), (39, 4)):
        idx = oracle.select(x[[t]], np.array([t]), refs, s, k)[0]
        assert np.all(idx[:k_eff] >= 0) and np.all(idx[k_eff:] == -1), (t, idx)
        assert len(set(idx[:k_eff].tolist())) == k_eff


def test_select_all_refs_equal_gives_lowest_ordinals():
    s, k = 3, 4
    x = np.full((30, 5), 2.0)
    x[1::3] = 1.0
    x[2::3] = -1.0
    refs = oracle.build_refs(x, s)
    pos = oracle.nonref_positions(30, s)
    idx = oracle.select(x[pos], pos, refs, s, k)
    for row, t in zip(idx, pos):
        k_eff = min(k, -(-int(t) // s))
        assert row.tolist() == list(range(k_eff)) + [-1] * (k - k_eff)


def test_select_is_causal():
    # the token just before a reference position must not see that reference,
    # the token just after it must
    rng = _rng(5)
    s, k = 4, 1
    x = rng.standard_normal((30, 6)) * 10
    x[11] = x[12] + 1e-3               # position 12 is ref 3
    x[13] = x[12] + 1e-3
    refs = oracle.build_refs(x, s)
    before = oracle.select(x[[11]], np.array([11]), refs, s, k)[0, 0]
    after = oracle.select(x[[13]], np.array([13]), refs, s, k)[0, 0]
    assert before != 3
    assert after == 3


def test_select_rejects_reference_positions():
    x = np.zeros((10, 2))
    with pytest.raises(ValueError):
        oracle.select(x[[4]], np.array([4]), oracle.build_refs(x, 2), 2, 1)


def test_sq_dist_is_ordered_sum_of_squares():
    a = np.array([1.0, -2.0, 3.5])
    b = np.array([0.5, 2.0, -1.0])
    assert oracle.sq_dist(a, b) == 0.25 + 16.0 + 20.25
    assert oracle.sq_dist(a, a) == 0.0


# ------------------------------------------------------------------------- GELU

def test_gelu_textbook_values():
    with open(os.path.join(GOLDEN, "std_normal_cdf.json")) as f:
        table = json.load(f)["values"]
    for e in table:
        x, phi = e["x"], e["phi"]
        assert abs(oracle.gelu(x) - x * phi) <= 1e-14 * max(1.0, abs(x))


def test_gelu_limits():
    assert oracle.gelu(0.0) == 0.0
    assert abs(oracle.gelu(12.0) - 12.0) < 1e-15
    assert abs(oracle.gelu(-12.0)) < 1e-30
    for u in np.linspace(-6, 6, 49):
        # GELU(u) - GELU(-u) = u (Phi(u) + Phi(-u) = 1)
        assert abs(oracle.gelu(u) - oracle.gelu(-u) - u) < 1e-14


# -------------------------------------------------------------------------- MLP

def _np_mlp(inp, m):
    h = inp @ m.w1.T + m.b1
    if m.act == ACT_GELU:
        h = 0.5 * h * (1 + scipy.special.erf(h / np.sqrt(2)))
    return h @ m.w2.T + m.b2


@pytest.mark.parametrize("act", [ACT_GELU, ACT_IDENTITY])
def test_mlp_matches_numpy_and_scipy(act):
    rng = _rng(11)
    m = MLP(rng.standard_normal((48, 20)) * 0.3, rng.standard_normal(48),
            rng.standard_normal((7, 48)) * 0.2, rng.standard_normal(7), act)
    inp = rng.standard_normal((33, 20)) * 3
    got = oracle.mlp(inp, m)
    want = _np_mlp(inp, m)
    assert got.shape == (33, 7)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


# ------------------------------------------------------------ compress / rebuild

def test_compress_mean_and_residual_closed_form():
    rng = _rng(12)
    d, k = 6, 4
    r = rng.standard_normal(d)
    refs = np.stack([r, r, r, r, r])
    xt = rng.standard_normal((3, d))
    idx = np.array([[0, 1, 2, 3], [4, 2, -1, -1], [3, -1, -1, -1]], np.int32)
    eye = MLP(np.eye(d), None, np.eye(d), None, ACT_IDENTITY)
    lat, kvr, res = oracle.compress(xt, refs, idx, eye)
    assert np.array_equal(kvr, np.tile(r, (3, 1)))
    assert np.array_equal(res, xt - r)
    assert np.array_equal(lat, xt - r)


def test_compress_mean_over_existing_refs_only():
    d = 3
    refs = np.array([[1.0, 2.0, 3.0], [3.0, 2.0, 1.0], [2.0, 8.0, -4.0]])
    idx = np.array([[2, 0, 1, -1]], np.int32)
    xt = np.zeros((1, d))
    eye = MLP(np.eye(d), None, np.eye(d), None, ACT_IDENTITY)
    _, kvr, res = oracle.compress(xt, refs, idx, eye)
    assert np.allclose(kvr[0], [2.0, 4.0, 0.0], rtol=0, atol=1e-15)
    assert np.allclose(res[0], [-2.0, -4.0, 0.0], rtol=0, atol=1e-15)


def test_compress_and_reconstruct_match_numpy_composition():
    rng = _rng(13)
    T, d, s, k, dc, h = 70, 12, 4, 3, 5, 16
    x = rng.standard_normal((T, d)) * 4
    comp = MLP(rng.standard_normal((h, d)) * 0.3, rng.standard_normal(h) * 0.1,
               rng.standard_normal((dc, h)) * 0.3, rng.standard_normal(dc) * 0.1)
    dec = MLP(rng.standard_normal((h, dc)) * 0.3, rng.standard_normal(h) * 0.1,
              rng.standard_normal((d, h)) * 0.3, rng.standard_normal(d) * 0.1)
    refs, idx, lat = oracle.compress_head(x, s, k, comp)
    pos = oracle.nonref_positions(T, s)
    kvr = np.stack([refs[row[row >= 0]].mean(axis=0) for row in idx])
    want_lat = _np_mlp(x[pos] - kvr, comp)
    assert np.max(np.abs(lat - want_lat)) <= 1e-12 * np.max(np.abs(want_lat))
    xhat = oracle.reconstruct(refs, lat, idx, T, s, dec)
    want = np.empty_like(x)
    want[::s] = x[::s]
    want[pos] = kvr + _np_mlp(lat, dec)
    assert np.max(np.abs(xhat - want)) <= 1e-12 * np.max(np.abs(want))


def _orthogonal_pair(d, seed):
    q, _ = np.linalg.qr(_rng(seed).standard_normal((d, d)))
    comp = MLP(q, None, np.eye(d), None, ACT_IDENTITY)
    dec = MLP(q.T, None, np.eye(d), None, ACT_IDENTITY)
    return comp, dec


@pytest.mark.parametrize("d,s,k", [(64, 16, 4), (32, 8, 8), (16, 3, 2)])
def test_orthogonal_pair_reconstructs_exactly(d, s, k):
    # with an orthogonal linear Compressor / Decompressor pair and d_c = head_dim
    # the rebuilt rows are the input rows (up to fp64 rounding)
    from deltakv_synth import kv_rows
    x = kv_rows(300, d, 4, 32, key=(9, d, s, k)).double().numpy()
    comp, dec = _orthogonal_pair(d, 21)
    refs, idx, lat = oracle.compress_head(x, s, k, comp)
    xhat = oracle.reconstruct(refs, lat, idx, 300, s, dec)
    assert np.max(np.abs(xhat - x)) <= 1e-12 * np.max(np.abs(x))


# ------------------------------------------------------------------- attention

def test_attention_matches_torch_sdpa_fp64():
    rng = _rng(14)
    G, T, d = 4, 257, 32
    q = rng.standard_normal((G, d))
    kk = rng.standard_normal((T, d)) * 2
    vv = rng.standard_normal((T, d))
    scale = 1 / np.sqrt(d)
    got = oracle.attention(q, kk, vv, scale)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kk)[None], torch.from_numpy(vv)[None],
        scale=scale)[0].numpy()
    assert np.max(np.abs(got - want)) <= 1e-12


def test_attention_scale_is_applied():
    rng = _rng(15)
    q = rng.standard_normal((2, 8))
    kk = rng.standard_normal((30, 8))
    vv = rng.standard_normal((30, 8))
    got = oracle.attention(q, kk, vv, 0.7)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kk)[None], torch.from_numpy(vv)[None],
        scale=0.7)[0].numpy()
    assert np.max(np.abs(got - want)) <= 1e-12


def test_attention_zero_query_is_mean_of_values():
    rng = _rng(16)
    vv = rng.standard_normal((50, 8))
    got = oracle.attention(np.zeros((1, 8)), rng.standard_normal((50, 8)), vv, 0.3)
    assert np.max(np.abs(got[0] - vv.mean(axis=0))) <= 1e-14


def test_decode_with_orthogonal_pair_is_dense_attention():
    from deltakv_synth import kv_rows
    T, d, s, k = 200, 32, 8, 4
    kx = kv_rows(T, d, 4, 16, key=(10, 0)).double().numpy()
    vx = kv_rows(T, d, 4, 16, key=(10, 1)).double().numpy()
    comp, dec = _orthogonal_pair(d, 5)
    kr, ki, kl = oracle.compress_head(kx, s, k, comp)
    vr, vi, vl = oracle.compress_head(vx, s, k, comp)
    q = _rng(17).standard_normal((4, d))
    scale = 1 / np.sqrt(d)
    got = oracle.decode_head(q, kr, kl, ki, dec, vr, vl, vi, dec, T, s, scale)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kx)[None], torch.from_numpy(vx)[None],
        scale=scale)[0].numpy()
    assert np.max(np.abs(got - want)) <= 1e-10 * np.max(np.abs(want))


# ------------------------------------------------- on-demand (sparse) rebuild

def _gelu_pair(rng, d, dc, h):
    comp = MLP(rng.standard_normal((h, d)) * 0.3, rng.standard_normal(h) * 0.1,
               rng.standard_normal((dc, h)) * 0.3, rng.standard_normal(dc) * 0.1)
    dec = MLP(rng.standard_normal((h, dc)) * 0.3, rng.standard_normal(h) * 0.1,
              rng.standard_normal((d, h)) * 0.3, rng.standard_normal(d) * 0.1)
    return comp, dec


def _sdpa64(q, kk, vv, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kk)[None], torch.from_numpy(vv)[None],
        scale=scale)[0].numpy()


def _np_rebuild(refs, lat, idx, T, s, dec, decoded=None):
    """Rows of one head rebuilt by NumPy: reference positions copy their row;
    every other position is the mean of its listed references plus the
    Decompressor's output (or plus `decoded`, a closed form of that output)."""
    pos = np.array([t for t in range(T) if t % s], dtype=np.int64)
    out = np.empty((T, refs.shape[1]))
    out[::s] = refs[:len(range(0, T, s))]
    kvr = np.stack([refs[row[row >= 0]].mean(axis=0) for row in idx])
    out[pos] = kvr + (_np_mlp(lat, dec) if decoded is None else decoded)
    return out


def _gelu_decode_case(seed, T=150, d=16, s=6, k=3, dc=5, h=24, G=3):
    rng = _rng(seed)
    kx = rng.standard_normal((T, d)) * 2
    vx = rng.standard_normal((T, d))
    kcomp, kdec = _gelu_pair(rng, d, dc, h)
    vcomp, vdec = _gelu_pair(rng, d, dc, h)
    kc = oracle.compress_head(kx, s, k, kcomp)
    vc = oracle.compress_head(vx, s, k, vcomp)
    q = rng.standard_normal((G, d))
    return T, d, s, q, kc, kdec, vc, vdec


def test_decode_with_gelu_weights_matches_numpy_rebuild_and_sdpa():
    # random GELU Decompressors: the oracle's decode equals fp64 SDPA over rows
    # rebuilt by NumPy matmuls and scipy's erf
    T, d, s, q, (kr, ki, kl), kdec, (vr, vi, vl), vdec = _gelu_decode_case(31)
    scale = 1 / np.sqrt(d)
    got = oracle.decode_head(q, kr, kl, ki, kdec, vr, vl, vi, vdec, T, s, scale)
    want = _sdpa64(q, _np_rebuild(kr, kl, ki, T, s, kdec),
                   _np_rebuild(vr, vl, vi, T, s, vdec), scale)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


@pytest.mark.parametrize("regime", ["off", "linear"])
def test_decode_gelu_saturated_decompressor_closed_forms(regime):
    # GELU(u) = u * Phi(u): with every hidden pre-activation pushed far below zero
    # it is 0 in fp64 (Phi(-60) underflows), so each rebuilt row is KV_R + b2;
    # pushed far above zero Phi is 1, the Decompressor is affine, and each row is
    # KV_R + W2 (W1 latent + b1) + b2
    T, d, s, q, (kr, ki, kl), kdec, (vr, vi, vl), vdec = _gelu_decode_case(32)
    shift = -60.0 if regime == "off" else 60.0
    kdec = MLP(kdec.w1, kdec.b1 + shift, kdec.w2, kdec.b2, ACT_GELU)
    vdec = MLP(vdec.w1, vdec.b1 + shift, vdec.w2, vdec.b2, ACT_GELU)
    for lat, m in ((kl, kdec), (vl, vdec)):
        pre = lat @ m.w1.T + m.b1
        assert (np.max(pre) < -40) if regime == "off" else (np.min(pre) > 40)

    def closed(lat, m):
        if regime == "off":
            return np.broadcast_to(m.b2, (len(lat), len(m.b2)))
        return (lat @ m.w1.T + m.b1) @ m.w2.T + m.b2

    scale = 0.4
    got = oracle.decode_head(q, kr, kl, ki, kdec, vr, vl, vi, vdec, T, s, scale)
    khat = _np_rebuild(kr, kl, ki, T, s, kdec, closed(kl, kdec))
    vhat = _np_rebuild(vr, vl, vi, T, s, vdec, closed(vl, vdec))
    want = _sdpa64(q, khat, vhat, scale)
    assert np.max(np.abs(got - want)) <= 1e-11 * np.max(np.abs(want))


@pytest.mark.parametrize("d,s,k", [(32, 16, 4), (16, 5, 3), (16, 1, 2)])
def test_reconstruct_at_identity_pair_gives_input_rows(d, s, k):
    # any order, references and compressed tokens mixed, repeats allowed
    from deltakv_synth import kv_rows
    T = 260
    x = kv_rows(T, d, 4, 16, key=(31, d, s, k)).double().numpy()
    comp, dec = _orthogonal_pair(d, 23)
    refs, idx, lat = oracle.compress_head(x, s, k, comp)
    pos = np.concatenate([_rng(32).integers(0, T, 90), [0, T - 1, s, s + 1, 1, 1]])
    got = oracle.reconstruct_at(refs, lat, idx, pos, s, dec)
    assert np.max(np.abs(got - x[pos])) <= 1e-12 * np.max(np.abs(x))


def test_reconstruct_at_matches_numpy_composition_by_searched_ordinal():
    # the latent / index row of a compressed position is found here by searching
    # the sorted list of non-reference positions, not by the oracle's closed form
    rng = _rng(33)
    T, d, s, k, dc, h = 150, 12, 6, 3, 5, 16
    x = rng.standard_normal((T, d)) * 3
    comp, dec = _gelu_pair(rng, d, dc, h)
    refs, idx, lat = oracle.compress_head(x, s, k, comp)
    nonref = oracle.nonref_positions(T, s)
    pos = rng.integers(0, T, 70)
    got = oracle.reconstruct_at(refs, lat, idx, pos, s, dec)
    for i, p in enumerate(pos):
        if p % s == 0:
            want = refs[p // s]
        else:
            q = int(np.searchsorted(nonref, p))
            assert nonref[q] == p
            row = idx[q][idx[q] >= 0]
            want = refs[row].mean(axis=0) + _np_mlp(lat[q:q + 1], dec)[0]
        assert np.max(np.abs(got[i] - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
    full = oracle.reconstruct(refs, lat, idx, T, s, dec)
    assert np.max(np.abs(got - full[pos])) <= 1e-13 * np.max(np.abs(full))


def _sparse_setup(seed, T=180, d=16, s=8, k=4, dc=6, h=16, G=3):
    rng = _rng(seed)
    kx = rng.standard_normal((T, d)) * 2
    vx = rng.standard_normal((T, d))
    comp, kdec = _gelu_pair(rng, d, dc, h)
    _, vdec = _gelu_pair(rng, d, dc, h)
    kr, ki, kl = oracle.compress_head(kx, s, k, comp)
    vr, vi, vl = oracle.compress_head(vx, s, k, comp)
    q = rng.standard_normal((G, d))
    args = (kr, kl, ki, kdec, vr, vl, vi, vdec, T, s, 1 / np.sqrt(d))
    return rng, q, args


def test_sparse_decode_over_every_position_is_the_dense_decode():
    rng, q, args = _sparse_setup(34)
    T = args[8]
    dense = oracle.decode_head(q, *args)
    got = oracle.decode_head_sparse(q, *args, rng.permutation(T))
    assert np.max(np.abs(got - dense)) <= 1e-12 * np.max(np.abs(dense))


def test_sparse_decode_with_identity_pair_is_attention_over_selected_rows():
    from deltakv_synth import kv_rows
    T, d, s, k = 240, 32, 8, 4
    kx = kv_rows(T, d, 4, 16, key=(35, 0)).double().numpy()
    vx = kv_rows(T, d, 4, 16, key=(35, 1)).double().numpy()
    comp, dec = _orthogonal_pair(d, 36)
    kr, ki, kl = oracle.compress_head(kx, s, k, comp)
    vr, vi, vl = oracle.compress_head(vx, s, k, comp)
    q = _rng(37).standard_normal((4, d))
    pos = np.sort(_rng(38).choice(T, 50, replace=False))
    scale = 1 / np.sqrt(d)
    got = oracle.decode_head_sparse(q, kr, kl, ki, dec, vr, vl, vi, dec, T, s, scale, pos)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kx[pos])[None],
        torch.from_numpy(vx[pos])[None], scale=scale)[0].numpy()
    assert np.max(np.abs(got - want)) <= 1e-10 * np.max(np.abs(want))


def test_sparse_decode_order_and_padding_do_not_matter():
    rng, q, args = _sparse_setup(39)
    T = args[8]
    pos = rng.choice(T, 40, replace=False)
    base = oracle.decode_head_sparse(q, *args, pos)
    shuffled = oracle.decode_head_sparse(q, *args, rng.permutation(pos))
    padded = oracle.decode_head_sparse(q, *args, np.concatenate([[-1, T, T + 7], pos, [-5]]))
    assert np.max(np.abs(shuffled - base)) <= 1e-13 * np.max(np.abs(base))
    assert np.array_equal(padded, base)


def test_sparse_decode_repeated_position_weighs_twice():
    # listing a position twice is attention with that row's logit raised by ln 2
    rng, q, args = _sparse_setup(40)
    kr, kl, ki, kdec, vr, vl, vi, vdec, T, s, scale = args
    pos = rng.choice(T, 30, replace=False)
    got = oracle.decode_head_sparse(q, *args, np.concatenate([pos, pos[:1]]))
    kh = oracle.reconstruct_at(kr, kl, ki, pos, s, kdec)
    vh = oracle.reconstruct_at(vr, vl, vi, pos, s, vdec)
    bias = torch.zeros(1, len(pos), dtype=torch.float64)
    bias[0, 0] = np.log(2.0)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kh)[None], torch.from_numpy(vh)[None],
        attn_mask=bias[None], scale=scale)[0].numpy()
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_sparse_decode_single_position_returns_its_value_row():
    rng, q, args = _sparse_setup(41)
    kr, kl, ki, kdec, vr, vl, vi, vdec, T, s, scale = args
    for p in (0, 1, s, T - 1):
        got = oracle.decode_head_sparse(q, *args, [p])
        vrow = oracle.reconstruct_at(vr, vl, vi, [p], s, vdec)[0]
        assert np.max(np.abs(got - vrow[None])) <= 1e-14 * max(1.0, np.max(np.abs(vrow)))


def test_sparse_decode_with_nothing_selected_is_zero():
    rng, q, args = _sparse_setup(42)
    T = args[8]
    assert np.array_equal(oracle.decode_head_sparse(q, *args, [-1, T]), np.zeros_like(q))


# ------------------------------------------------ query-aware token selection

def test_group_attention_mass_matches_torch_softmax_and_sums_to_group_size():
    rng = _rng(50)
    G, T, d = 4, 300, 16
    q = rng.standard_normal((G, d))
    kk = rng.standard_normal((T, d)) * 2
    got = oracle.group_attention_mass(q, kk, 0.25)
    want = torch.softmax(torch.from_numpy(q) @ torch.from_numpy(kk).T * 0.25, dim=1).sum(0)
    assert np.max(np.abs(got - want.numpy())) <= 1e-13
    assert abs(got.sum() - G) <= 1e-12


def _rule_by_tuples(scores, n_keep):
    # the rule written out with Python's tuple order
    ranked = sorted(range(len(scores)), key=lambda t: (-float(scores[t]), t))
    if n_keep >= len(scores):
        return list(range(len(scores))) + [-1] * (n_keep - len(scores))
    return sorted(ranked[:n_keep])


@pytest.mark.parametrize("seed", range(8))
def test_top_positions_matches_tuple_sort_with_ties(seed):
    rng = _rng(60 + seed)
    T = int(rng.integers(1, 80))
    # few distinct values: many exact ties, including at the cut
    scores = rng.integers(0, 5, T).astype(np.float32) / 4
    for n_keep in (1, max(1, T // 3), T - 1 if T > 1 else 1, T, T + 5):
        assert list(oracle.top_positions(scores, n_keep)) == _rule_by_tuples(scores, n_keep)


def test_select_head_with_identity_pair_ranks_the_input_rows():
    # with the orthogonal identity pair the rebuilt keys are the input rows,
    # so the selection is the rule applied to softmax weights over x
    from deltakv_synth import kv_rows
    T, d, s, k = 200, 32, 8, 4
    kx = kv_rows(T, d, 4, 16, key=(51, 0)).double().numpy()
    comp, dec = _orthogonal_pair(d, 52)
    kr, ki, kl = oracle.compress_head(kx, s, k, comp)
    q = _rng(53).standard_normal((4, d))
    scale = 1 / np.sqrt(d)
    pos, mass = oracle.select_head(q, kr, kl, ki, dec, T, s, scale, 37)
    want_mass = torch.softmax(torch.from_numpy(q) @ torch.from_numpy(kx).T * scale, 1).sum(0)
    assert np.max(np.abs(mass - want_mass.numpy())) <= 1e-10
    assert list(pos) == _rule_by_tuples(want_mass.numpy(), 37)


def test_select_head_equal_keys_prefer_the_lower_position():
    # two tokens with the same rebuilt key get the same mass; the cut between
    # them keeps the lower position
    rng = _rng(54)
    T, d = 40, 8
    kk = rng.standard_normal((T, d))
    q = rng.standard_normal((2, d))
    mass0 = oracle.group_attention_mass(q, kk, 1.0)
    top = int(np.argmax(mass0))
    kk[T - 1] = kk[top]          # a later copy of the best key
    mass = oracle.group_attention_mass(q, kk, 1.0)
    assert mass[T - 1] == mass[top]
    assert list(oracle.top_positions(mass, 1)) == [min(top, T - 1)]


# ---------------------------------------------------------- 4-bit latents

def _bf16_rows(rng, n, dc, scale=1.0):
    return torch.from_numpy(rng.standard_normal((n, dc)) * scale).to(torch.bfloat16).float().numpy()


def test_bf16_rounding_helper_matches_torch():
    x = _rng(70).standard_normal(5000).astype(np.float32) * 100
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle._bf16_round(x), want)


def _bf16_exact(v: Fraction) -> Fraction:
    """Nearest bf16 value to the rational v (8 significant bits, step 2^-133
    below 2^-126), ties to the even significand, in exact arithmetic."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1                                                   # 2^e <= a < 2^(e+1)
    step = Fraction(2) ** max(e - 7, -133)
    return round(v / step) * step                                # round(): half to even


def test_bf16_from_f64_is_exact_rounding_including_near_midpoints():
    rng = _rng(73)
    x = rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000)
    # values just off a bf16 midpoint: rounding through fp32 first lands on
    # the midpoint and then goes to the even neighbour, which is wrong for
    # half of them; the helper must round once
    base = oracle._bf16_round(rng.standard_normal(400).astype(np.float32) * 4).astype(np.float64)
    _, e = np.frexp(base)
    mid = base + np.ldexp(1.0, e - 9)
    off = np.concatenate([mid + np.ldexp(1.0, e - 40), mid - np.ldexp(1.0, e - 40), mid])
    x = np.concatenate([x, off, [0.0, -0.0, 2.0 ** -130, 3.0 * 2.0 ** -134]])
    got = oracle.bf16_from_f64(x)
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == _bf16_exact(Fraction(float(xi))), xi
    via_f32 = oracle._bf16_round(off.astype(np.float32)).astype(np.float64)
    assert np.any(via_f32 != oracle.bf16_from_f64(off)), "expected double rounding to differ"


def _quantize_exact(zrow):
    """The 4-bit format in exact rational arithmetic (an independent
    implementation): scale = bf16((max - min) / 15), code = nearest integer to
    (z - min) / scale, half to even, clamped to 0..15."""
    zf = [Fraction(float(v)) for v in zrow]
    lo = min(zf)
    scale = _bf16_exact((max(zf) - lo) / 15)
    if scale == 0:
        return [0] * len(zf), lo, scale, [None] * len(zf)
    quo = [(v - lo) / scale for v in zf]
    return [min(15, max(0, round(q))) for q in quo], lo, scale, quo


def test_quantized_latents_equal_exact_rational_definition():
    rng = _rng(74)
    rows = [_bf16_rows(rng, 150, 32, 3.0), _bf16_rows(rng, 150, 16, 1e-3),
            # magnitudes far apart in one row (small values beside large ones)
            _bf16_rows(rng, 100, 32, 1.0) * (10.0 ** rng.integers(-12, 3, (100, 32)))]
    near_ties = exact_ties = 0
    for z in rows:
        z = torch.from_numpy(z).to(torch.bfloat16).double().numpy()
        codes, shift, scale = oracle.quantize_latents(z)
        for i in range(z.shape[0]):
            c, lo, sc, quo = _quantize_exact(z[i])
            assert Fraction(float(shift[i])) == lo and Fraction(float(scale[i])) == sc, i
            for j in range(z.shape[1]):
                gap = None if quo[j] is None else \
                    abs(quo[j] - round(quo[j] - Fraction(1, 2)) - Fraction(1, 2))
                if gap is not None and 0 < gap < Fraction(1, 2 ** 40):
                    near_ties += 1   # fp64 may resolve such a quotient either way
                    continue
                exact_ties += gap == 0
                assert codes[i, j] == c[j], (i, j, z[i, j])
    assert near_ties == 0 and exact_ties > 0


def test_quantized_half_integer_quotients_go_to_the_even_code():
    # scale 1/4 (range 15/4), entries at shift + (n + 1/2) / 4: every quotient
    # is an exact half-integer and every value is exact in bf16
    for shift in (0.0, -2.0, 1.5):
        n = np.arange(15)
        z = np.concatenate([[shift, shift + 3.75], shift + (n + 0.5) * 0.25])[None, :]
        z = np.concatenate([z, z[:, :16]], axis=1)[:, :32]
        assert np.array_equal(oracle._bf16_round(z.astype(np.float32)), z.astype(np.float32))
        codes, sh, sc = oracle.quantize_latents(z)
        assert sc[0] == 0.25 and sh[0] == shift
        want = np.concatenate([[0, 15], 2 * np.round((n + 0.5) / 2)])   # even neighbour
        want = np.concatenate([want, want[:16]])[:32]
        assert np.array_equal(codes[0], want.astype(np.uint8))
        assert list(codes[0, 2:7]) == [0, 2, 2, 4, 4]


@pytest.mark.parametrize("dc", [16, 32])
def test_quantized_latents_within_half_a_step(dc):
    z = _bf16_rows(_rng(71), 500, dc, 3.0)
    codes, shift, scale = oracle.quantize_latents(z)
    assert codes.dtype == np.uint8 and codes.max() <= 15
    zh = oracle.dequantize_latents(codes, shift, scale)
    # scale is rounded to bf16 (relative error <= 2^-9); the clamp at 15 can
    # add that rounding times 15 at the top of the range
    bound = scale[:, None] * (0.5 + 15 * 2.0 ** -8) + 1e-30
    assert np.all(np.abs(zh - z) <= bound)
    assert np.all(codes[np.arange(500), z.argmin(1)] == 0)
    assert np.all(codes[np.arange(500), z.argmax(1)] >= 14)
    assert np.array_equal(shift, z.min(1))


def test_quantized_latents_recover_rows_built_from_codes():
    # rows that are exactly shift + code * scale with min code 0 and max 15
    rng = _rng(72)
    n, dc = 200, 32
    codes = rng.integers(0, 16, (n, dc)).astype(np.uint8)
    codes[:, 0], codes[:, 1] = 0, 15
    shift = torch.from_numpy(rng.standard_normal(n)).to(torch.bfloat16).float().numpy()
    scale = np.float32(2.0) ** rng.integers(-6, 2, n).astype(np.float32)  # exact in bf16
    z = (shift[:, None] + codes.astype(np.float32) * scale[:, None]).astype(np.float32)
    z = oracle._bf16_round(z)
    keep = np.all(oracle.dequantize_latents(codes, shift, scale) == z, axis=1)  # rows exact in bf16
    c2, s2, k2 = oracle.quantize_latents(z[keep])
    assert keep.sum() > 50
    assert np.array_equal(c2, codes[keep]) and np.array_equal(k2, scale[keep])


def test_quantized_constant_rows_are_exact():
    z = np.full((4, 16), -1.5, np.float32)
    codes, shift, scale = oracle.quantize_latents(z)
    assert np.all(codes == 0) and np.all(scale == 0)
    assert np.array_equal(oracle.dequantize_latents(codes, shift, scale), z.astype(np.float64))


# ------------------------------------------ exact rows beside the compressed cache

def test_window_decode_with_identity_pair_is_attention_over_rows_and_window():
    from deltakv_synth import kv_rows
    T, d, s, k, W = 200, 32, 8, 4, 37
    kx = kv_rows(T + W, d, 4, 16, key=(80, 0)).double().numpy()
    vx = kv_rows(T + W, d, 4, 16, key=(80, 1)).double().numpy()
    comp, dec = _orthogonal_pair(d, 81)
    kr, ki, kl = oracle.compress_head(kx[:T], s, k, comp)
    vr, vi, vl = oracle.compress_head(vx[:T], s, k, comp)
    q = _rng(82).standard_normal((4, d))
    scale = 1 / np.sqrt(d)
    got = oracle.decode_head_window(q, kr, kl, ki, dec, vr, vl, vi, dec, T, s, scale,
                                    kx[T:], vx[T:])
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kx)[None], torch.from_numpy(vx)[None],
        scale=scale)[0].numpy()
    assert np.max(np.abs(got - want)) <= 1e-10 * np.max(np.abs(want))


def test_window_decode_weighs_a_repeated_row_twice_and_ignores_window_order():
    rng, q, args = _sparse_setup(83)
    kr, kl, ki, kdec, vr, vl, vi, vdec, T, s, scale = args
    d = kr.shape[1]
    kw = rng.standard_normal((9, d))
    vw = rng.standard_normal((9, d))
    base = oracle.decode_head_window(q, *args, kw, vw)
    perm = rng.permutation(9)
    assert np.max(np.abs(oracle.decode_head_window(q, *args, kw[perm], vw[perm]) - base)) <= \
        1e-13 * np.max(np.abs(base))
    # repeating window row 0 = attention with its logit raised by ln 2
    rep = oracle.decode_head_window(q, *args, np.vstack([kw, kw[:1]]), np.vstack([vw, vw[:1]]))
    kh = np.vstack([oracle.reconstruct(kr, kl, ki, T, s, kdec), kw])
    vh = np.vstack([oracle.reconstruct(vr, vl, vi, T, s, vdec), vw])
    bias = torch.zeros(1, T + 9, dtype=torch.float64)
    bias[0, T] = np.log(2.0)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(kh)[None], torch.from_numpy(vh)[None],
        attn_mask=bias[None], scale=scale)[0].numpy()
    assert np.max(np.abs(rep - want)) <= 1e-12 * np.max(np.abs(want))
