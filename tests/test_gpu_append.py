"""GPU parity of the batched one-token append (deltakv_append).

A decode step appends one token to every layer's K and V cache.  The batched
entry point must leave every cache bit for bit as the per-cache calls
deltakv_build_refs(t, t + 1) + deltakv_compress(t, t + 1) would, for
reference positions (a verbatim copy) and compressed ones (exact top-k over the
references so far, then the Compressor), and over more caches than one
launch set holds.  The appended tokens are also checked against the oracle:
reference rows bitwise, index lists exactly, latents to the path's tolerance."""
import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
from parity import (TOL, check_compress_unit, gpu_mlp, make_kv, make_mlp, oracle_mlp, say)

pytestmark = pytest.mark.gpu


def _same(a, b, n_refs, n_toks, q4, dc):
    """Equal bytes over the filled prefix of every array of two caches."""
    assert torch.equal(a.refs[:, :, :n_refs].view(torch.int16),
                       b.refs[:, :, :n_refs].view(torch.int16)) if a.refs.dtype == torch.bfloat16 \
        else torch.equal(a.refs[:, :, :n_refs], b.refs[:, :, :n_refs])
    assert torch.equal(a.ref_sqnorm[:, :, :n_refs].view(torch.int32),
                       b.ref_sqnorm[:, :, :n_refs].view(torch.int32))
    if n_toks:
        assert torch.equal(a.idx[:, :, :n_toks].view(torch.int16),
                           b.idx[:, :, :n_toks].view(torch.int16))
        if q4:
            assert torch.equal(a.latent_codes[:, :, :n_toks], b.latent_codes[:, :, :n_toks])
            assert torch.equal(a.latent_params[:, :, :n_toks].view(torch.int16),
                               b.latent_params[:, :, :n_toks].view(torch.int16))
        else:
            la, lb = a.latents[:, :, :n_toks], b.latents[:, :, :n_toks]
            assert torch.equal(la.view(torch.int16), lb.view(torch.int16)) \
                if la.dtype == torch.bfloat16 else torch.equal(la, lb)


def _append_case(name, n_items, B, H, d, s, k, dc, hid, dtype, T0, A, seed, q4=False,
                 oracle_items=(0,), acts=None):
    say(f"[case] {name}: items={n_items} B={B} H={H} d={d} s={s} k={k} dc={dc} hid={hid} "
        f"dtype={dtype} T0={T0} A={A} q4={q4}")
    tdt = torch.float32 if dtype == dk.F32 else torch.bfloat16
    cap = T0 + A
    shape = dk.Shape(B, H, d, s, k, dc, cap, dtype, dk.LATENT_Q4 if q4 else 0)
    xs = [make_kv(B, H, cap, d, tdt, key=(seed, i)) for i in range(n_items)]
    mlps = [make_mlp(d, hid, dc, tdt, key=(seed, 100 + i), bias_std=0.05)[0]
            for i in range(n_items)]
    acts = acts or [dk.ACT_GELU] * n_items
    comps = [gpu_mlp(w, acts[i]) for i, w in enumerate(mlps)]
    xg = [x.cuda() for x in xs]
    ref_c = [dk.Cache(shape) for _ in range(n_items)]
    bat_c = [dk.Cache(shape) for _ in range(n_items)]
    # the prompt, per cache, into both sets
    ws = dk.workspace(max(dk.compress_workspace_bytes(shape, 0, T0),
                          dk.compress_workspace_bytes(shape, cap - 1, cap)))
    for i in range(n_items):
        xp = xg[i][:, :, :T0].contiguous()
        for c in (ref_c[i], bat_c[i]):
            dk.build_refs(shape, xp, 0, T0, c)
            dk.compress(shape, xp, 0, T0, comps[i], c, ws)
    # the appended rows, one [B, H, 1, d] tensor per (position, cache)
    rows = [[xg[i][:, :, t:t + 1].contiguous() for i in range(n_items)] for t in range(cap)]
    aws = dk.workspace(dk.append_workspace_bytes(shape, cap - 1, n_items))
    batch = dk.AppendBatch(shape, bat_c, comps)
    aws.fill_(0xFF)
    for t in range(T0, cap):
        for i in range(n_items):
            dk.build_refs(shape, rows[t][i], t, t + 1, ref_c[i])
            dk.compress(shape, rows[t][i], t, t + 1, comps[i], ref_c[i], ws)
        batch(t, rows[t], aws)
    torch.cuda.synchronize()
    n_refs = -(-cap // s)
    n_toks = cap - n_refs
    for i in range(n_items):
        assert bat_c[i].n_built == bat_c[i].n_compressed == cap
        _same(ref_c[i], bat_c[i], n_refs, n_toks, q4, dc)
    # the appended positions of a few caches against the oracle
    pos = np.array([p for p in range(T0, cap) if p % s])
    err = 0.0
    if not q4:
        for i in oracle_items:
            for b in range(B):
                for h in range(H):
                    err = max(err, check_compress_unit(shape, xs[i][b, h], bat_c[i], b, h,
                                                       oracle_mlp(mlps[i], acts[i]),
                                                       positions=pos, tol=TOL[dtype]))
    say(f"[case] {name}: bitwise equal to the per-cache calls over {n_items} caches, "
        f"{A} appends; appended latent rel err {err:.3e}")


def test_append_layers_and_streams_stride8_k8():
    # the streaming shapes (stride 8, k 8, d_c 16, hidden 256), three layers x
    # K and V, 21 appends crossing three reference positions
    _append_case("append-s8k8", 6, 1, 2, 128, 8, 8, 16, 256, dk.BF16, T0=611, A=21, seed=501,
                 oracle_items=(0, 5))


def test_append_more_caches_than_one_launch_set():
    # 40 caches: two launch sets of the batched kernels
    _append_case("append-40", 40, 1, 1, 64, 16, 4, 32, 128, dk.BF16, T0=200, A=18, seed=502,
                 oracle_items=(0, 39))


def test_append_k_beyond_the_references_so_far():
    # early positions have fewer than k candidates (unused slots 0xFFFF)
    _append_case("append-early", 4, 2, 2, 128, 4, 8, 32, 256, dk.BF16, T0=1, A=30, seed=503,
                 oracle_items=(1,))


def test_append_q4_latents():
    _append_case("append-q4", 4, 1, 2, 128, 8, 8, 16, 256, dk.BF16, T0=300, A=12, seed=504,
                 q4=True)


@pytest.mark.parametrize("cfg", [
    (3, 1, 2, 64, 5, 3, 16, 64, dk.BF16),     # hidden 64: per-cache launches inside the call
    (3, 1, 2, 64, 8, 4, 16, 128, dk.F32),     # fp32 storage
    (2, 1, 2, 128, 16, 4, 128, 256, dk.BF16),  # d_c 128
], ids=["hidden64", "fp32", "dc128"])
def test_append_shapes_outside_the_batched_kernels(cfg):
    n, B, H, d, s, k, dc, hid, dtype = cfg
    _append_case(f"append-{cfg}", n, B, H, d, s, k, dc, hid, dtype, T0=150, A=11, seed=505,
                 oracle_items=range(n))


def test_append_mixed_activations():
    # compressors that differ in activation cannot share one launch set: the
    # call falls back to per-cache launches, with the same result
    acts = [dk.ACT_GELU, dk.ACT_IDENTITY, dk.ACT_GELU]
    _append_case("append-mixed-act", 3, 1, 2, 128, 8, 8, 16, 256, dk.BF16, T0=100, A=9,
                 seed=506, oracle_items=(0, 1), acts=acts)
