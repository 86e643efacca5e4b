"""GPU check of deltakv_decode_attn_noalloc, the decode entry point that
allocates nothing (its scratch is a device array inside the library).  Two
calls in a row through the C ABI, the second over a shorter context, each
compared with deltakv_decode_attn (the caller's workspace) on the same inputs:
both run the same kernels with the same launch plan, so the outputs must be
equal bit for bit; the first call is also checked against the oracle on one KV
head (max over rows of max|g - o| / max|o| <= 2e-2, bf16)."""
import math

import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
from deltakv_synth import queries
from parity import (TOL, gpu_compress, gpu_mlp, make_kv, make_mlp, oracle_decode_head,
                    oracle_mlp, rel_err_rows, say, to_np)

pytestmark = pytest.mark.gpu


def test_noalloc_decode_equals_workspace_decode_on_two_calls_second_smaller():
    B, H, G, T, d, s, k, dc, hid = 1, 4, 4, 3000, 128, 16, 4, 32, 256
    say(f"[case] noalloc: B={B} H={H} G={G} T={T}, then 1100 tokens")
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    kx = make_kv(B, H, T, d, torch.bfloat16, key=(801, 0))
    vx = make_kv(B, H, T, d, torch.bfloat16, key=(801, 1))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(801, 10), bias_std=0.05)
    kc = gpu_compress(shape, kx, gpu_mlp(cw, dk.ACT_GELU))
    vc = gpu_compress(shape, vx, gpu_mlp(cw, dk.ACT_GELU))
    kdw, _ = make_mlp(dc, hid, d, torch.bfloat16, key=(801, 12), bias_std=0.05)
    vdw, _ = make_mlp(dc, hid, d, torch.bfloat16, key=(801, 13), bias_std=0.05)
    kd, vd = gpu_mlp(kdw, dk.ACT_GELU), gpu_mlp(vdw, dk.ACT_GELU)
    Hq, scale = H * G, 1.0 / math.sqrt(d)
    q = queries(B * Hq, d, key=(801, 20), dtype=torch.bfloat16).reshape(B, Hq, d).cuda()
    for n_tok in (T, 1100):
        ws = dk.workspace(dk.decode_workspace_bytes(shape, Hq, n_tok))
        out_ws = torch.full((B, Hq, d), float("nan"), device="cuda")
        out_na = torch.full((B, Hq, d), float("nan"), device="cuda")
        dk.decode_attn(shape, Hq, n_tok, q, kc, kd, vc, vd, scale, out_ws, ws)
        dk.decode_attn_noalloc(shape, Hq, n_tok, q, kc, kd, vc, vd, scale, out_na)
        torch.cuda.synchronize()
        assert torch.isfinite(out_na).all()
        assert torch.equal(out_na, out_ws), f"{n_tok} tokens: outputs differ"
        h = 2
        want = oracle_decode_head(shape, n_tok, to_np(q[0, h * G:(h + 1) * G].cpu()), kc, vc, 0,
                                  h, oracle_mlp(kdw, dk.ACT_GELU), oracle_mlp(vdw, dk.ACT_GELU),
                                  scale)
        err = rel_err_rows(out_na[0, h * G:(h + 1) * G].cpu().double().numpy(), want)
        say(f"[case] noalloc {n_tok} tokens: bitwise equal to the workspace call, "
            f"oracle rel err {err:.3e}")
        assert err <= TOL[dk.BF16]
