"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the CPU oracle on the same inputs, compare."""
import math
import sys

import numpy as np
import torch

import decode_attention_deltakv_amd as dk
import oracle
from deltakv_synth import kv_rows, xavier_mlp, queries

TOL = {dk.F32: 1e-4, dk.BF16: 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err_rows(got, want):
    """max over rows of max_i |g - o| / max_i |o| (rows = last axis)."""
    got = np.asarray(got, np.float64).reshape(-1, np.shape(want)[-1])
    want = np.asarray(want, np.float64).reshape(-1, np.shape(want)[-1])
    den = np.maximum(np.abs(want).max(axis=1), 1e-30)
    return float((np.abs(got - want).max(axis=1) / den).max())


def to_np(t):
    return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else \
        t.detach().cpu().double().numpy()


def idx_to_oracle(idx_u16):
    a = idx_u16.cpu().numpy().astype(np.int64) if isinstance(idx_u16, torch.Tensor) else idx_u16
    a = a.astype(np.int64)
    a[a == 0xFFFF] = -1
    return a.astype(np.int32)


def make_kv(B, H, T, d, dtype, key, n_dirs=8, n_centroids=64):
    x = torch.empty(B, H, T, d, dtype=dtype)
    for b in range(B):
        for h in range(H):
            x[b, h] = kv_rows(T, d, n_dirs, n_centroids, key=key + (b, h), dtype=dtype)
    return x


def make_mlp(din, hid, dout, dtype, key, bias_std=0.0, act=dk.ACT_GELU):
    w = xavier_mlp(din, hid, dout, key=key, dtype=dtype, bias_std=bias_std)
    return w, act


def gpu_mlp(w, act):
    return dk.Mlp(w["w1"].cuda(), w["b1"].cuda(), w["w2"].cuda(), w["b2"].cuda(), act)


def oracle_mlp(w, act):
    return oracle.MLP(to_np(w["w1"]), w["b1"].double().numpy(), to_np(w["w2"]),
                      w["b2"].double().numpy(), act)


def gpu_compress(shape, x_cpu, comp, chunks=None, stats=None):
    """Build + compress positions [0, T) of x ([B, H, T, d], CPU) on the GPU, in
    one call or in the given chunk boundaries. Returns the device cache."""
    T = x_cpu.shape[2]
    cache = dk.Cache(shape)
    bounds = [0, T] if chunks is None else chunks
    xg = x_cpu.cuda()
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        xc = xg[:, :, t0:t1].contiguous()
        dk.build_refs(shape, xc, t0, t1, cache)
        ws = dk.workspace(dk.compress_workspace_bytes(shape, t0, t1))
        dk.compress(shape, xc, t0, t1, comp, cache, ws, stats)
    torch.cuda.synchronize()
    return cache


def gpu_decode(shape, Hq, T, q_cpu, kc, kdec, vc, vdec, scale):
    out = torch.empty(shape.batch, Hq, shape.head_dim, dtype=torch.float32, device="cuda")
    ws = dk.workspace(dk.decode_workspace_bytes(shape, Hq, T))
    dk.decode_attn(shape, Hq, T, q_cpu.cuda(), kc, kdec, vc, vdec, scale, out, ws)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def check_compress_unit(shape, x_unit, cache, b, h, comp_o, positions=None, tol=None):
    """Oracle vs GPU for one unit: refs bitwise, idx exact, latents to tol.
    Returns the latent relative error."""
    s, k = shape.stride, shape.k
    T = x_unit.shape[0]
    xo = to_np(x_unit)
    R = oracle.num_refs(T, s)
    g_refs = cache.refs[b, h, :R].cpu()
    assert torch.equal(g_refs.view(torch.int16) if g_refs.dtype == torch.bfloat16 else
                       g_refs.view(torch.int32),
                       x_unit[::s].view(torch.int16) if x_unit.dtype == torch.bfloat16 else
                       x_unit[::s].view(torch.int32)), "reference rows not copied verbatim"
    refs_o = oracle.build_refs(xo, s)
    pos = oracle.nonref_positions(T, s) if positions is None else np.asarray(positions)
    if len(pos) == 0:
        return 0.0
    qord = (pos // s) * (s - 1) + (pos % s) - 1
    idx_o = oracle.select(xo[pos], pos, refs_o, s, k)
    idx_g = idx_to_oracle(cache.idx[b, h].cpu()[torch.from_numpy(qord)])
    bad = np.nonzero((idx_g != idx_o).any(axis=1))[0]
    assert len(bad) == 0, (f"idx mismatch at {len(bad)} tokens, first position "
                           f"{pos[bad[0]]}: gpu {idx_g[bad[0]]} oracle {idx_o[bad[0]]}")
    lat_o, _, _ = oracle.compress(xo[pos], refs_o, idx_o, comp_o)
    lat_g = to_np(cache.latents[b, h].cpu()[torch.from_numpy(qord)])
    err = rel_err_rows(lat_g, lat_o)
    if tol is not None:
        assert err <= tol, f"latent rel err {err} > {tol}"
    return err


def oracle_decode_head(shape, T, q_rows, kc, vc, b, h, kdec_o, vdec_o, scale):
    """Oracle attention for the query rows of KV head (b, h), rebuilt from the
    GPU's stored cache (refs, latents, idx)."""
    s = shape.stride
    R = oracle.num_refs(T, s)
    N = T - R

    def grab(c):
        refs = to_np(c.refs[b, h, :R].cpu())
        lat = to_np(c.latents[b, h, :N].cpu()) if N > 0 else np.zeros((0, shape.d_c))
        idx = idx_to_oracle(c.idx[b, h, :N].cpu()) if N > 0 else np.zeros((0, shape.k),
                                                                           np.int32)
        return refs, lat, idx

    kr, kl, ki = grab(kc)
    vr, vl, vi = grab(vc)
    return oracle.decode_head(q_rows, kr, kl, ki, kdec_o, vr, vl, vi, vdec_o, T, s, scale)


def check_selection(scores_g, kept_g, mass_o, n_keep, eps):
    """The selection of one (sequence, KV head) against the oracle's attention
    masses mass_o [T] (fp64, rebuilt keys):
      - scores, position by position: |g_p - o_p| <= eps * max(o_p, floor),
        floor = 1e-3 * tau, tau = the oracle's n_keep-th largest mass (the
        selection threshold), so every position near the cut is held to the
        relative bound;
      - the kept positions are a valid top n_keep of the oracle's masses up to
        that bound: with e_p = eps * max(o_p, floor), a kept p and a dropped
        p' can be in the wrong order only if o_p + e_p >= o_p' - e_p', which
        bounds every kept o_p >= tau (1 - 3 eps) - 2 eps floor and every
        dropped o_p <= tau (1 + 3 eps) + 2 eps floor.
    Returns (largest per-position relative error, positions kept by exactly
    one of the two sides)."""
    o = np.asarray(mass_o, np.float64)
    g = np.asarray(scores_g, np.float64)
    T = len(o)
    kept = np.asarray(kept_g)
    kept = kept[kept >= 0]
    tau = np.sort(o)[::-1][min(n_keep, T) - 1]
    floor = 1e-3 * tau
    den = np.maximum(o, floor)
    rel = np.abs(g - o) / den
    worst = float(rel.max())
    assert worst <= eps, (f"score at position {int(rel.argmax())}: gpu {g[rel.argmax()]:.6e} "
                          f"oracle {o[rel.argmax()]:.6e} (rel {worst:.3e} > {eps})")
    if n_keep >= T:
        assert np.array_equal(np.sort(kept), np.arange(T)), "n_keep >= T must keep everything"
        return worst, 0
    assert len(kept) == n_keep and len(np.unique(kept)) == n_keep
    mask = np.zeros(T, bool)
    mask[kept] = True
    lo = tau * (1 - 3 * eps) - 2 * eps * floor
    hi = tau * (1 + 3 * eps) + 2 * eps * floor
    assert o[mask].min() >= lo, f"kept position with oracle mass {o[mask].min():.6e} < {lo:.6e}"
    if (~mask).any():
        assert o[~mask].max() <= hi, (f"dropped position with oracle mass {o[~mask].max():.6e} "
                                      f"> {hi:.6e}")
    ref = np.zeros(T, bool)
    ref[np.lexsort((np.arange(T), -o))[:n_keep]] = True
    return worst, int((mask != ref).sum())
