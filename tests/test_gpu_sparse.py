"""GPU parity of the sparse decode (on-demand reconstruction of the listed
positions only) against the CPU oracle, on the GPU's own stored cache.

Each unit (sequence, KV head) gets its own seeded position list mixing
compressed tokens and references in random order, with padding entries
outside [0, T), repeated positions, a list of references only, a list of
compressed tokens only and an empty list (zero output).  Tolerances as for
the dense decode: max over rows of max|g - o| / max|o| <= 2e-2 (bf16),
1e-4 (fp32)."""
import math

import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
import oracle
from deltakv_synth import kv_rows, queries
from parity import (TOL, gpu_compress, gpu_decode, gpu_mlp, idx_to_oracle, make_kv, make_mlp,
                    oracle_mlp, rel_err_rows, say, to_np)

pytestmark = pytest.mark.gpu


def _unit_list(rng, T, s, n_sel, kind):
    """One unit's position list of length n_sel (int32, padding = -1 / >= T)."""
    refs = np.arange(0, T, s)
    comp = np.setdiff1d(np.arange(T), refs)
    if kind == "empty":
        return np.where(rng.random(n_sel) < 0.5, -1, T + rng.integers(0, 50, n_sel))
    if kind == "refs":
        pool = refs
    elif kind == "comp":
        pool = comp if len(comp) else refs
    else:
        pool = np.arange(T)
    n_real = max(1, int(n_sel * 0.8))
    pick = rng.choice(pool, min(n_real, len(pool)), replace=False)
    extra = n_sel - len(pick)
    # repeats of picked positions, then padding, then a shuffle
    rep = rng.choice(pick, extra // 2) if extra // 2 else np.zeros(0, np.int64)
    pad = np.full(extra - len(rep), -1)
    pad[1::2] = T + 3
    lst = np.concatenate([pick, rep, pad])
    rng.shuffle(lst)
    return lst


def _grab(c, b, h, R, N, shape):
    refs = to_np(c.refs[b, h, :R].cpu())
    lat = to_np(c.latents[b, h, :N].cpu()) if N > 0 else np.zeros((0, shape.d_c))
    idx = idx_to_oracle(c.idx[b, h, :N].cpu()) if N > 0 else np.zeros((0, shape.k), np.int32)
    return refs, lat, idx


def _sparse_case(name, B, H, G, T, d, s, k, dc, hid, dtype, seed, n_sel, kinds=None,
                 heads=None, lists=None, caches=None):
    say(f"[case] {name}: B={B} H={H} G={G} T={T} d={d} s={s} k={k} dc={dc} hid={hid} "
        f"dtype={dtype} seed={seed} n_sel={n_sel}")
    tdt = torch.float32 if dtype == dk.F32 else torch.bfloat16
    shape = dk.Shape(B, H, d, s, k, dc, T, dtype)
    if caches is None:
        kx = make_kv(B, H, T, d, tdt, key=(seed, 0))
        vx = make_kv(B, H, T, d, tdt, key=(seed, 1))
        kcw, _ = make_mlp(d, hid, dc, tdt, key=(seed, 10), bias_std=0.05)
        kc = gpu_compress(shape, kx, gpu_mlp(kcw, dk.ACT_GELU))
        vc = gpu_compress(shape, vx, gpu_mlp(kcw, dk.ACT_GELU))
    else:
        kc, vc = caches
    kdw, _ = make_mlp(dc, hid, d, tdt, key=(seed, 12), bias_std=0.05)
    vdw, _ = make_mlp(dc, hid, d, tdt, key=(seed, 13), bias_std=0.05)
    rng = np.random.default_rng(seed)
    if lists is None:
        kinds = kinds or ["mixed"] * (B * H)
        lists = np.stack([_unit_list(rng, T, s, n_sel, kinds[u % len(kinds)])
                          for u in range(B * H)]).reshape(B, H, n_sel)
    pos = torch.from_numpy(lists.astype(np.int32)).cuda()
    Hq = H * G
    q = queries(B * Hq, d, key=(seed, 20), dtype=tdt).reshape(B, Hq, d)
    scale = 1.0 / math.sqrt(d)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = dk.workspace(dk.decode_sparse_workspace_bytes(shape, Hq, T, n_sel))
    ws.fill_(0xFF)  # stale workspace content must not leak into the result
    dk.decode_attn_sparse(shape, Hq, T, q.cuda(), kc, gpu_mlp(kdw, dk.ACT_GELU), vc,
                          gpu_mlp(vdw, dk.ACT_GELU), pos, scale, out, ws)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    R = oracle.num_refs(T, s)
    N = T - R
    err = 0.0
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in heads:
        kr, kl, ki = _grab(kc, b, h, R, N, shape)
        vr, vl, vi = _grab(vc, b, h, R, N, shape)
        want = oracle.decode_head_sparse(to_np(q[b, h * G:(h + 1) * G]), kr, kl, ki,
                                         oracle_mlp(kdw, dk.ACT_GELU), vr, vl, vi,
                                         oracle_mlp(vdw, dk.ACT_GELU), T, s, scale, lists[b, h])
        got = out[b, h * G:(h + 1) * G]
        if not np.any(want):
            assert np.array_equal(got, want), f"unit ({b}, {h}): empty list must give zeros"
            continue
        err = max(err, rel_err_rows(got, want))
    say(f"[case] {name}: sparse decode rel err {err:.3e}")
    assert err <= TOL[dtype], f"sparse decode rel err {err} > {TOL[dtype]}"
    return shape, kc, vc, q, kdw, vdw, out


def test_sparse_fp32_general_path():
    _sparse_case("sparse-fp32-tiny", 1, 2, 2, 512, 64, 16, 4, 16, 128, dk.F32, seed=301,
                 n_sel=100, kinds=["mixed", "refs"])


def test_sparse_bf16_mixed_lists_padding_repeats_and_empty():
    _sparse_case("sparse-bf16-mixed", 2, 2, 4, 1000, 128, 16, 4, 32, 256, dk.BF16, seed=302,
                 n_sel=300, kinds=["mixed", "refs", "comp", "empty"])


@pytest.mark.parametrize("cfg", [
    # (B, H, G, T, d, s, k, dc, hid, dtype, n_sel)
    (1, 2, 4, 1500, 128, 8, 8, 16, 256, dk.BF16, 400),
    (1, 2, 8, 900, 64, 5, 3, 64, 128, dk.BF16, 257),
    (1, 1, 1, 700, 64, 7, 6, 16, 64, dk.F32, 333),
    (2, 1, 4, 333, 128, 16, 4, 128, 128, dk.BF16, 64),
], ids=["k8-dc16", "d64-k3-dc64-G8", "fp32-k6-h64", "bf16-dc128-general"])
def test_sparse_shape_variants(cfg):
    B, H, G, T, d, s, k, dc, hid, dtype, n_sel = cfg
    _sparse_case(f"sparse-{cfg}", B, H, G, T, d, s, k, dc, hid, dtype, seed=303 + n_sel,
                 n_sel=n_sel)


def test_sparse_many_partitions_and_reference_blocks():
    # every reference (1250 > one 512-row reference block) plus 3000 compressed
    # tokens: several token partitions and three reference partitions
    B, H, T, s = 1, 2, 20000, 16
    rng = np.random.default_rng(304)
    comp = np.setdiff1d(np.arange(T), np.arange(0, T, s))
    lists = []
    for _ in range(B * H):
        lst = np.concatenate([np.arange(0, T, s), rng.choice(comp, 3000, replace=False)])
        rng.shuffle(lst)
        lists.append(lst)
    lists = np.stack(lists).reshape(B, H, -1)
    _sparse_case("sparse-many-partitions", B, H, 4, T, 128, s, 4, 32, 256, dk.BF16, seed=304,
                 n_sel=lists.shape[-1], lists=lists)


@pytest.mark.parametrize("dtype", [dk.F32, dk.BF16])
def test_sparse_over_every_position_matches_dense_decode(dtype):
    B, H, G, T, d, s, k, dc, hid = 1, 2, 4, 600, 64, 16, 4, 16, 128
    rng = np.random.default_rng(305)
    lists = np.stack([rng.permutation(T) for _ in range(B * H)]).reshape(B, H, T)
    shape, kc, vc, q, kdw, vdw, out = _sparse_case(
        f"sparse-all-positions-{dtype}", B, H, G, T, d, s, k, dc, hid, dtype, seed=305, n_sel=T,
        lists=lists)
    dense = gpu_decode(shape, H * G, T, q, kc, gpu_mlp(kdw, dk.ACT_GELU), vc,
                       gpu_mlp(vdw, dk.ACT_GELU), 1.0 / math.sqrt(d))
    assert rel_err_rows(out, dense) <= TOL[dtype]


def test_sparse_llama_layer_128k_sampled_heads():
    # one Llama-3.1-8B-shaped layer at 128k context, compressed on the GPU from
    # inputs generated there; 4096 sorted random positions per KV head (the
    # launch the benchmark times); the oracle checks two KV heads
    B, H, G, T, d, s, k, dc, hid = 1, 8, 4, 131072, 128, 16, 4, 32, 256
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    say("[case] sparse-llama-128k: generating and compressing")
    kx = torch.stack([kv_rows(T, d, 8, 1024, key=(306, 0, h), dtype=torch.bfloat16,
                              device="cuda") for h in range(H)])[None]
    vx = torch.stack([kv_rows(T, d, 8, 1024, key=(306, 1, h), dtype=torch.bfloat16,
                              device="cuda") for h in range(H)])[None]
    kcw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(306, 10))
    caches = []
    for x in (kx, vx):
        cache = dk.Cache(shape)
        dk.build_refs(shape, x, 0, T, cache)
        ws = dk.workspace(dk.compress_workspace_bytes(shape, 0, T))
        dk.compress(shape, x, 0, T, gpu_mlp(kcw, dk.ACT_GELU), cache, ws)
        caches.append(cache)
    torch.cuda.synchronize()
    del kx, vx
    rng = np.random.default_rng(306)
    lists = np.stack([np.sort(rng.choice(T, 4096, replace=False)) for _ in range(H)])[None]
    _sparse_case("sparse-llama-128k", B, H, G, T, d, s, k, dc, hid, dk.BF16, seed=306,
                 n_sel=4096, lists=lists, heads=[(0, 0), (0, 5)], caches=tuple(caches))
