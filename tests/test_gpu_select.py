"""GPU parity of the dense decode with query-aware token selection.

Checks, on the GPU's own stored cache:
  - the attention output is bitwise the plain dense decode's;
  - the per-position scores (attention mass summed over the KV head's query
    heads) are within the path's tolerance of the oracle's (fp64, rebuilt
    keys) position by position, relative to each mass (2e-2 bf16, 1e-4
    fp32; floor 1e-3 of the selection threshold);
  - the positions are exactly what the selection rule (largest scores, ties
    to the lower position, in position order) gives on the GPU's own fp32
    scores -- the ranking is integer work on values both sides share;
  - the kept set is a valid top n_keep of the oracle's masses: every kept
    position's oracle mass is at least the oracle's threshold less the score
    bound, every dropped one's at most the threshold plus it;
  - each head's scores sum to its group size.
The three decode kernels (wave-specialised, matrix-core, general) are all
covered, with ties forced at the cut and n_keep >= n_tokens."""
import math

import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
import oracle
from deltakv_synth import queries
from parity import (TOL, check_selection, gpu_compress, gpu_decode, gpu_mlp, idx_to_oracle,
                    make_kv, make_mlp, oracle_mlp, rel_err_rows, say, to_np)

pytestmark = pytest.mark.gpu


def _select_case(name, B, H, G, T, d, s, k, dc, hid, dtype, seed, n_keep, heads=None,
                 kx=None, then_sparse=False):
    say(f"[case] {name}: B={B} H={H} G={G} T={T} d={d} s={s} k={k} dc={dc} hid={hid} "
        f"dtype={dtype} seed={seed} n_keep={n_keep}")
    tdt = torch.float32 if dtype == dk.F32 else torch.bfloat16
    shape = dk.Shape(B, H, d, s, k, dc, T, dtype)
    if kx is None:
        kx = make_kv(B, H, T, d, tdt, key=(seed, 0))
    vx = make_kv(B, H, T, d, tdt, key=(seed, 1))
    cw, _ = make_mlp(d, hid, dc, tdt, key=(seed, 10), bias_std=0.05)
    kc = gpu_compress(shape, kx, gpu_mlp(cw, dk.ACT_GELU))
    vc = gpu_compress(shape, vx, gpu_mlp(cw, dk.ACT_GELU))
    kdw, _ = make_mlp(dc, hid, d, tdt, key=(seed, 12), bias_std=0.05)
    vdw, _ = make_mlp(dc, hid, d, tdt, key=(seed, 13), bias_std=0.05)
    Hq = H * G
    q = queries(B * Hq, d, key=(seed, 20), dtype=tdt).reshape(B, Hq, d)
    scale = 1.0 / math.sqrt(d)
    kd, vd = gpu_mlp(kdw, dk.ACT_GELU), gpu_mlp(vdw, dk.ACT_GELU)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    pos = torch.full((B, H, n_keep), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, H, T), float("nan"), dtype=torch.float32, device="cuda")
    ws = dk.workspace(dk.decode_select_workspace_bytes(shape, Hq, T))
    ws.fill_(0xFF)
    dk.decode_attn_select(shape, Hq, T, q.cuda(), kc, kd, vc, vd, scale, out, pos, sc, ws)
    torch.cuda.synchronize()
    dense = gpu_decode(shape, Hq, T, q, kc, kd, vc, vd, scale)
    assert np.array_equal(out.cpu().double().numpy(), dense), "output differs from dense decode"
    pos_g = pos.cpu().numpy()
    sc_g = sc.cpu().numpy()
    assert np.all(np.isfinite(sc_g))
    R = oracle.num_refs(T, s)
    N = T - R
    err = 0.0
    for b in range(B):
        for h in range(H):
            want_pos = oracle.top_positions(sc_g[b, h], n_keep)
            assert np.array_equal(pos_g[b, h], want_pos), f"selection differs at unit ({b}, {h})"
            assert abs(float(sc_g[b, h].astype(np.float64).sum()) - G) <= 1e-3 * G
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    differ = 0
    for b, h in heads:
        refs = to_np(kc.refs[b, h, :R].cpu())
        lat = to_np(kc.latents[b, h, :N].cpu()) if N else np.zeros((0, dc))
        idx = idx_to_oracle(kc.idx[b, h, :N].cpu()) if N else np.zeros((0, k), np.int32)
        _, mass = oracle.select_head(to_np(q[b, h * G:(h + 1) * G]), refs, lat, idx,
                                     oracle_mlp(kdw, dk.ACT_GELU), T, s, scale, n_keep)
        e, dif = check_selection(sc_g[b, h], pos_g[b, h], mass, n_keep, TOL[dtype])
        err, differ = max(err, e), differ + dif
    say(f"[case] {name}: per-position score rel err {err:.3e}; kept sets differ from the "
        f"oracle's ranking at {differ} positions (within the score bound)")
    if then_sparse:
        # the selection feeds the sparse decode of the same layer
        sws = dk.workspace(dk.decode_sparse_workspace_bytes(shape, Hq, T, n_keep))
        sout = torch.empty_like(out)
        dk.decode_attn_sparse(shape, Hq, T, q.cuda(), kc, kd, vc, vd, pos, scale, sout, sws)
        torch.cuda.synchronize()
        sout = sout.cpu().double().numpy()
        for b, h in heads:
            kr = to_np(kc.refs[b, h, :R].cpu()); vr = to_np(vc.refs[b, h, :R].cpu())
            kl = to_np(kc.latents[b, h, :N].cpu()); vl = to_np(vc.latents[b, h, :N].cpu())
            ki = idx_to_oracle(kc.idx[b, h, :N].cpu()); vi = idx_to_oracle(vc.idx[b, h, :N].cpu())
            want = oracle.decode_head_sparse(to_np(q[b, h * G:(h + 1) * G]), kr, kl, ki,
                                             oracle_mlp(kdw, dk.ACT_GELU), vr, vl, vi,
                                             oracle_mlp(vdw, dk.ACT_GELU), T, s, scale,
                                             pos_g[b, h])
            assert rel_err_rows(sout[b, h * G:(h + 1) * G], want) <= TOL[dtype]
    return pos_g, sc_g


def test_select_wave_specialised_path_feeds_sparse_decode():
    _select_case("select-bf16-ws", 2, 2, 4, 1000, 128, 16, 4, 32, 256, dk.BF16, seed=401,
                 n_keep=100, then_sparse=True)


@pytest.mark.parametrize("cfg", [
    # (B, H, G, T, d, s, k, dc, hid, dtype, n_keep)
    (1, 2, 4, 700, 64, 5, 3, 64, 128, dk.BF16, 64),      # matrix-core kernel (k = 3)
    (1, 2, 2, 512, 64, 16, 4, 16, 128, dk.F32, 50),      # general kernel (fp32)
    (1, 1, 8, 900, 128, 8, 8, 16, 256, dk.BF16, 300),    # wave-specialised, k = 8, G = 8
    (1, 2, 4, 333, 128, 16, 4, 32, 256, dk.BF16, 333),   # n_keep = T: everything
    (1, 2, 4, 333, 128, 16, 4, 32, 256, dk.BF16, 400),   # n_keep > T: padded with -1
    (1, 2, 4, 300, 128, 16, 4, 32, 256, dk.BF16, 1),
], ids=["mfma-k3", "fp32-general", "ws-k8-G8", "keep-all", "keep-more", "keep-one"])
def test_select_shape_variants(cfg):
    B, H, G, T, d, s, k, dc, hid, dtype, n_keep = cfg
    pos, _ = _select_case(f"select-{cfg}", B, H, G, T, d, s, k, dc, hid, dtype,
                          seed=402 + n_keep, n_keep=n_keep)
    if n_keep >= T:
        assert np.array_equal(pos[0, 0, :T], np.arange(T)) and np.all(pos[0, 0, T:] == -1)


def test_select_ties_at_the_cut_go_to_the_lower_position():
    # every K row equal: every reference gets the same logit, and so do the
    # compressed tokens that share a reference count, so the cut falls inside
    # runs of exactly equal scores
    B, H, G, T, d, s = 1, 2, 4, 400, 128, 16
    row = make_kv(1, 1, 1, d, torch.bfloat16, key=(403, 0))[0, 0, 0]
    kx = row.expand(B, H, T, d).contiguous()
    pos, sc = _select_case("select-ties", B, H, G, T, d, s, 4, 32, 256, dk.BF16, seed=403,
                           n_keep=37, kx=kx)
    assert len(np.unique(sc[0, 0])) < T // 4, "expected many equal scores"


def test_select_llama_layer_32k_two_heads():
    # the one-layer Llama-3.1-8B-shaped workload: 4096 of 32768 positions kept
    # per KV head; scores checked against the oracle on two heads
    _select_case("select-llama-32k", 1, 8, 4, 32768, 128, 16, 4, 32, 256, dk.BF16, seed=404,
                 n_keep=4096, heads=[(0, 0), (0, 6)])


def test_sparse_and_select_calls_replay_in_a_graph():
    # both calls captured in one HIP graph (fresh queries copied in before each
    # replay); every replay must equal the eager calls bitwise
    B, H, G, T, d, s, k, dc, hid = 1, 2, 4, 900, 128, 16, 4, 32, 256
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    kx = make_kv(B, H, T, d, torch.bfloat16, key=(405, 0))
    vx = make_kv(B, H, T, d, torch.bfloat16, key=(405, 1))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(405, 10))
    kc = gpu_compress(shape, kx, gpu_mlp(cw, dk.ACT_GELU))
    vc = gpu_compress(shape, vx, gpu_mlp(cw, dk.ACT_GELU))
    kd = gpu_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(405, 12))[0], dk.ACT_GELU)
    vd = gpu_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(405, 13))[0], dk.ACT_GELU)
    Hq, n_keep, scale = H * G, 120, 1.0 / math.sqrt(d)
    qbank = [queries(B * Hq, d, key=(405, 20 + i), dtype=torch.bfloat16).reshape(B, Hq, d).cuda()
             for i in range(4)]
    qbuf = qbank[0].clone()
    pos = torch.empty(B, H, n_keep, dtype=torch.int32, device="cuda")
    out_sel = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    out_sp = torch.empty_like(out_sel)
    sws = dk.workspace(dk.decode_select_workspace_bytes(shape, Hq, T))
    pws = dk.workspace(dk.decode_sparse_workspace_bytes(shape, Hq, T, n_keep))

    def step():
        dk.decode_attn_select(shape, Hq, T, qbuf, kc, kd, vc, vd, scale, out_sel, pos, None, sws)
        dk.decode_attn_sparse(shape, Hq, T, qbuf, kc, kd, vc, vd, pos, scale, out_sp, pws)

    want = []
    for qi in qbank:
        qbuf.copy_(qi)
        step()
        torch.cuda.synchronize()
        want.append((out_sel.clone(), pos.clone(), out_sp.clone()))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, qi in enumerate(qbank):
            qbuf.copy_(qi)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_sel, want[i][0]), f"replay {rep}.{i}: select output"
            assert torch.equal(pos, want[i][1]), f"replay {rep}.{i}: positions"
            assert torch.equal(out_sp, want[i][2]), f"replay {rep}.{i}: sparse output"
