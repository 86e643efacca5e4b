"""GPU parity of decode attention over the compressed cache plus exact window
rows (a recent window not yet compressed, or attention sinks), against the
CPU oracle on the GPU's stored cache: max over rows of max|g - o| / max|o| <=
2e-2 (bf16), 1e-4 (fp32)."""
import math

import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
import oracle
from deltakv_synth import queries
from parity import (TOL, gpu_compress, gpu_mlp, idx_to_oracle, make_kv, make_mlp, oracle_mlp,
                    rel_err_rows, say, to_np)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [
    # (B, H, G, T, n_win, d, s, k, dc, hid, dtype, latent_format)
    (2, 2, 4, 1000, 64, 128, 16, 4, 32, 256, dk.BF16, dk.LATENT_DTYPE),   # wave-specialised
    (1, 2, 4, 900, 1500, 128, 16, 4, 32, 256, dk.BF16, dk.LATENT_DTYPE),  # window > cache
    (1, 2, 2, 512, 1, 64, 16, 4, 16, 128, dk.F32, dk.LATENT_DTYPE),       # general, one row
    (1, 2, 8, 700, 300, 64, 5, 3, 64, 128, dk.BF16, dk.LATENT_DTYPE),     # matrix-core, k = 3
    (1, 2, 4, 800, 200, 128, 16, 4, 32, 256, dk.BF16, dk.LATENT_Q4),      # 4-bit latents
], ids=["ws", "long-window", "fp32-one-row", "mfma-k3", "q4"])
def test_window_decode_matches_oracle(cfg):
    B, H, G, T, W, d, s, k, dc, hid, dtype, lf = cfg
    seed = 601 + T + W
    say(f"[case] window {cfg}")
    tdt = torch.float32 if dtype == dk.F32 else torch.bfloat16
    shape = dk.Shape(B, H, d, s, k, dc, T, dtype, lf)
    kx = make_kv(B, H, T + W, d, tdt, key=(seed, 0))
    vx = make_kv(B, H, T + W, d, tdt, key=(seed, 1))
    cw, _ = make_mlp(d, hid, dc, tdt, key=(seed, 10), bias_std=0.05)
    kc = gpu_compress(shape, kx[:, :, :T].contiguous(), gpu_mlp(cw, dk.ACT_GELU))
    vc = gpu_compress(shape, vx[:, :, :T].contiguous(), gpu_mlp(cw, dk.ACT_GELU))
    kdw, _ = make_mlp(dc, hid, d, tdt, key=(seed, 12), bias_std=0.05)
    vdw, _ = make_mlp(dc, hid, d, tdt, key=(seed, 13), bias_std=0.05)
    Hq = H * G
    q = queries(B * Hq, d, key=(seed, 20), dtype=tdt).reshape(B, Hq, d)
    scale = 1.0 / math.sqrt(d)
    kw = kx[:, :, T:].contiguous().cuda()
    vw = vx[:, :, T:].contiguous().cuda()
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = dk.workspace(dk.decode_window_workspace_bytes(shape, Hq, T, W))
    ws.fill_(0xFF)
    dk.decode_attn_window(shape, Hq, T, q.cuda(), kc, gpu_mlp(kdw, dk.ACT_GELU), vc,
                          gpu_mlp(vdw, dk.ACT_GELU), kw, vw, scale, out, ws)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    R = oracle.num_refs(T, s)
    N = T - R
    err = 0.0
    for b in range(B):
        for h in range(H):
            def grab(c):
                refs = to_np(c.refs[b, h, :R].cpu())
                if lf == dk.LATENT_Q4:
                    cb = c.latent_codes[b, h, :N].cpu().numpy()
                    codes = np.empty((N, dc), np.uint8)
                    codes[:, 0::2], codes[:, 1::2] = cb & 15, cb >> 4
                    par = c.latent_params[b, h, :N].cpu().float().numpy()
                    lat = oracle.dequantize_latents(codes, par[:, 0], par[:, 1])
                else:
                    lat = to_np(c.latents[b, h, :N].cpu())
                return refs, lat, idx_to_oracle(c.idx[b, h, :N].cpu())
            kr, kl, ki = grab(kc)
            vr, vl, vi = grab(vc)
            want = oracle.decode_head_window(to_np(q[b, h * G:(h + 1) * G]), kr, kl, ki,
                                             oracle_mlp(kdw, dk.ACT_GELU), vr, vl, vi,
                                             oracle_mlp(vdw, dk.ACT_GELU), T, s, scale,
                                             to_np(kx[b, h, T:]), to_np(vx[b, h, T:]))
            err = max(err, rel_err_rows(out[b, h * G:(h + 1) * G], want))
    say(f"[case] window {cfg}: rel err {err:.3e}")
    assert err <= TOL[dtype], f"window decode rel err {err} > {TOL[dtype]}"
