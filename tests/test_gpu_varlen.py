"""GPU parity of decode attention over a batch of sequences of different
lengths: sequence b attends its first lengths[b] positions, checked against
the oracle's dense decode at that length on the GPU's stored cache (max over
rows of max|g - o| / max|o| <= 2e-2 bf16, 1e-4 fp32)."""
import math

import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
from deltakv_synth import queries
from parity import (TOL, gpu_compress, gpu_mlp, make_kv, make_mlp, oracle_decode_head,
                    oracle_mlp, rel_err_rows, say, to_np)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [
    # (lengths, G, d, s, k, dc, hid, dtype)
    ((1200, 517, 33, 1024), 4, 128, 16, 4, 32, 256, dk.BF16),   # wave-specialised
    ((640, 1, 17, 200), 2, 64, 16, 4, 16, 128, dk.F32),         # general
    ((900, 455), 8, 64, 5, 3, 64, 128, dk.BF16),                # matrix-core, k = 3
], ids=["bf16-ws", "fp32", "bf16-k3"])
def test_varlen_decode_matches_oracle_per_sequence(cfg):
    lengths, G, d, s, k, dc, hid, dtype = cfg
    B, H, T = len(lengths), 2, max(lengths)
    seed = 701 + T
    say(f"[case] varlen {cfg}")
    tdt = torch.float32 if dtype == dk.F32 else torch.bfloat16
    shape = dk.Shape(B, H, d, s, k, dc, T, dtype)
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
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = dk.workspace(dk.decode_varlen_workspace_bytes(shape, Hq, T))
    ws.fill_(0xFF)
    lens = torch.tensor(lengths, dtype=torch.int64, device="cuda")
    dk.decode_attn_varlen(shape, Hq, lens, T, q.cuda(), kc, gpu_mlp(kdw, dk.ACT_GELU), vc,
                          gpu_mlp(vdw, dk.ACT_GELU), scale, out, ws)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    err = 0.0
    for b, L in enumerate(lengths):
        for h in range(H):
            want = oracle_decode_head(shape, L, to_np(q[b, h * G:(h + 1) * G]), kc, vc, b, h,
                                      oracle_mlp(kdw, dk.ACT_GELU), oracle_mlp(vdw, dk.ACT_GELU),
                                      scale)
            err = max(err, rel_err_rows(out[b, h * G:(h + 1) * G], want))
    say(f"[case] varlen {cfg}: rel err {err:.3e}")
    assert err <= TOL[dtype], f"mixed-length decode rel err {err} > {TOL[dtype]}"


def test_varlen_lengths_change_between_graph_replays():
    # the lengths are a device array read by the kernels: one captured call
    # replays with new lengths (written into the same array) and must give,
    # bitwise, what an eager call with those lengths gives; a length above
    # max_tokens is taken as max_tokens, and one below 1 as 1
    B, H, G, T, d, s, k, dc, hid = 3, 2, 4, 900, 128, 16, 4, 32, 256
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    kx = make_kv(B, H, T, d, torch.bfloat16, key=(702, 0))
    vx = make_kv(B, H, T, d, torch.bfloat16, key=(702, 1))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(702, 10))
    kc = gpu_compress(shape, kx, gpu_mlp(cw, dk.ACT_GELU))
    vc = gpu_compress(shape, vx, gpu_mlp(cw, dk.ACT_GELU))
    kd = gpu_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(702, 12))[0], dk.ACT_GELU)
    vd = gpu_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(702, 13))[0], dk.ACT_GELU)
    Hq, scale = H * G, 1.0 / math.sqrt(d)
    q = queries(B * Hq, d, key=(702, 20), dtype=torch.bfloat16).reshape(B, Hq, d).cuda()
    ws = dk.workspace(dk.decode_varlen_workspace_bytes(shape, Hq, T))
    lens = torch.zeros(B, dtype=torch.int64, device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    sets = [(900, 17, 450), (1, 899, 32), (5000, -3, 640)]
    want = []
    for ls in sets:
        lens.copy_(torch.tensor(ls))
        dk.decode_attn_varlen(shape, Hq, lens, T, q, kc, kd, vc, vd, scale, out, ws)
        torch.cuda.synchronize()
        want.append(out.clone())
    # clamping: (5000, -3, 640) is (900, 1, 640)
    lens.copy_(torch.tensor((900, 1, 640)))
    dk.decode_attn_varlen(shape, Hq, lens, T, q, kc, kd, vc, vd, scale, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, want[2])
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dk.decode_attn_varlen(shape, Hq, lens, T, q, kc, kd, vc, vd, scale, out, ws)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            dk.decode_attn_varlen(shape, Hq, lens, T, q, kc, kd, vc, vd, scale, out, ws)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, ls in enumerate(sets):
            lens.copy_(torch.tensor(ls))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, want[i]), f"replay {rep}.{i}"
    # the first set against the oracle
    outn = want[0].cpu().double().numpy()
    for b, L in enumerate(sets[0]):
        for h in range(H):
            ref = oracle_decode_head(shape, L, to_np(q[b, h * G:(h + 1) * G].cpu()), kc, vc, b,
                                     h, oracle_mlp(make_mlp(dc, hid, d, torch.bfloat16,
                                                            key=(702, 12))[0], dk.ACT_GELU),
                                     oracle_mlp(make_mlp(dc, hid, d, torch.bfloat16,
                                                         key=(702, 13))[0], dk.ACT_GELU), scale)
            assert rel_err_rows(outn[b, h * G:(h + 1) * G], ref) <= TOL[dk.BF16]
