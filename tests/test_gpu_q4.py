"""GPU parity of 4-bit latent storage (codes plus a per-row bf16 shift and
scale) against the CPU oracle.

  - The same inputs are compressed twice, with latents stored in bf16 and in
    4 bits: the index lists must be identical, and the 4-bit codes, shifts and
    scales must equal, bit for bit, the oracle's quantisation of the bf16 run's
    latents (both sides quantise the same bf16 values by the format's fp64
    definition: integer codes decided in the same precision on both sides).
  - Decode (dense, sparse and with selection) over the 4-bit cache must match
    the oracle's attention over the dequantised latents within the bf16
    tolerance (2e-2).
  - Chunked (streaming) compression gives the offline bytes."""
import math

import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
import oracle
from deltakv_synth import queries
from parity import (TOL, check_selection, gpu_compress, gpu_mlp, idx_to_oracle, make_kv,
                    make_mlp, oracle_mlp, rel_err_rows, say, to_np)

pytestmark = pytest.mark.gpu


def _unpack(codes_u8):
    """[..., d_c / 2] bytes -> [..., d_c] codes (low nibble first)."""
    c = codes_u8.cpu().numpy()
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def _both(B, H, T, d, s, k, dc, hid, seed, chunks=None):
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    shape4 = dk.Shape(B, H, d, s, k, dc, T, dk.BF16, dk.LATENT_Q4)
    x = make_kv(B, H, T, d, torch.bfloat16, key=(seed, 0))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(seed, 10), bias_std=0.05)
    c16 = gpu_compress(shape, x, gpu_mlp(cw, dk.ACT_GELU), chunks)
    c4 = gpu_compress(shape4, x, gpu_mlp(cw, dk.ACT_GELU), chunks)
    return shape, shape4, x, cw, c16, c4


def _check_codes(shape, c16, c4):
    R = oracle.num_refs(shape.capacity, shape.stride)
    N = shape.capacity - R
    assert torch.equal(c16.idx[:, :, :N].cpu(), c4.idx[:, :, :N].cpu()), "index lists differ"
    assert torch.equal(c16.refs.cpu().view(torch.int16), c4.refs.cpu().view(torch.int16))
    for b in range(shape.batch):
        for h in range(shape.num_kv_heads):
            z = c16.latents[b, h, :N].cpu().float().numpy()
            codes, shift, scale = oracle.quantize_latents(z)
            got_c = _unpack(c4.latent_codes[b, h, :N])
            par = c4.latent_params[b, h, :N].cpu().float().numpy()
            bad = np.nonzero((got_c != codes).any(axis=1))[0]
            assert len(bad) == 0, (f"codes differ at {len(bad)} rows of unit ({b}, {h}); first "
                                   f"ordinal {bad[0]}: gpu {got_c[bad[0]]} oracle {codes[bad[0]]}")
            assert np.array_equal(par[:, 0], shift), "shifts differ"
            assert np.array_equal(par[:, 1], scale), "scales differ"


@pytest.mark.parametrize("cfg", [
    # (B, H, T, d, s, k, dc, hid)
    (2, 2, 1000, 128, 16, 4, 32, 256),
    (1, 2, 1500, 128, 8, 8, 16, 256),
    (1, 3, 777, 64, 16, 4, 16, 128),
], ids=["d128-k4-dc32", "d128-k8-dc16", "d64-dc16-h128"])
def test_q4_codes_are_the_oracle_quantisation_of_the_bf16_latents(cfg):
    B, H, T, d, s, k, dc, hid = cfg
    say(f"[case] q4-codes {cfg}")
    shape, shape4, x, cw, c16, c4 = _both(B, H, T, d, s, k, dc, hid, seed=501 + T)
    _check_codes(shape, c16, c4)


def test_q4_streaming_chunks_match_offline_bytes():
    B, H, T, d, s, k, dc, hid = 1, 2, 1200, 128, 16, 4, 32, 256
    shape4 = dk.Shape(B, H, d, s, k, dc, T, dk.BF16, dk.LATENT_Q4)
    x = make_kv(B, H, T, d, torch.bfloat16, key=(502, 0))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(502, 10), bias_std=0.05)
    off = gpu_compress(shape4, x, gpu_mlp(cw, dk.ACT_GELU))
    chk = gpu_compress(shape4, x, gpu_mlp(cw, dk.ACT_GELU), chunks=[0, 300, 301, 777, 1200])
    R = oracle.num_refs(T, s)
    N = T - R
    assert torch.equal(off.latent_codes[:, :, :N].cpu(), chk.latent_codes[:, :, :N].cpu())
    assert torch.equal(off.latent_params[:, :, :N].cpu().view(torch.int16),
                       chk.latent_params[:, :, :N].cpu().view(torch.int16))


def _oracle_cache(shape, c4, b, h):
    R = oracle.num_refs(shape.capacity, shape.stride)
    N = shape.capacity - R
    refs = to_np(c4.refs[b, h, :R].cpu())
    codes = _unpack(c4.latent_codes[b, h, :N])
    par = c4.latent_params[b, h, :N].cpu().float().numpy()
    lat = oracle.dequantize_latents(codes, par[:, 0], par[:, 1])
    return refs, lat, idx_to_oracle(c4.idx[b, h, :N].cpu())


@pytest.mark.parametrize("cfg", [
    # (B, H, G, T, d, s, k, dc, hid)
    (2, 2, 4, 1000, 128, 16, 4, 32, 256),
    (1, 2, 8, 1500, 128, 8, 8, 16, 256),
], ids=["k4-dc32-G4", "k8-dc16-G8"])
def test_q4_decode_dense_sparse_and_select_match_oracle(cfg):
    B, H, G, T, d, s, k, dc, hid = cfg
    seed = 503 + T
    say(f"[case] q4-decode {cfg}")
    shape4 = dk.Shape(B, H, d, s, k, dc, T, dk.BF16, dk.LATENT_Q4)
    kx = make_kv(B, H, T, d, torch.bfloat16, key=(seed, 0))
    vx = make_kv(B, H, T, d, torch.bfloat16, key=(seed, 1))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(seed, 10), bias_std=0.05)
    kc = gpu_compress(shape4, kx, gpu_mlp(cw, dk.ACT_GELU))
    vc = gpu_compress(shape4, vx, gpu_mlp(cw, dk.ACT_GELU))
    kdw, _ = make_mlp(dc, hid, d, torch.bfloat16, key=(seed, 12), bias_std=0.05)
    vdw, _ = make_mlp(dc, hid, d, torch.bfloat16, key=(seed, 13), bias_std=0.05)
    kd, vd = gpu_mlp(kdw, dk.ACT_GELU), gpu_mlp(vdw, dk.ACT_GELU)
    Hq = H * G
    q = queries(B * Hq, d, key=(seed, 20), dtype=torch.bfloat16).reshape(B, Hq, d)
    qg = q.cuda()
    scale = 1.0 / math.sqrt(d)
    # dense, and dense with selection
    out = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    ws = dk.workspace(dk.decode_workspace_bytes(shape4, Hq, T))
    dk.decode_attn(shape4, Hq, T, qg, kc, kd, vc, vd, scale, out, ws)
    n_keep = 150
    pos = torch.empty(B, H, n_keep, dtype=torch.int32, device="cuda")
    sc = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
    out_sel = torch.empty_like(out)
    sws = dk.workspace(dk.decode_select_workspace_bytes(shape4, Hq, T))
    dk.decode_attn_select(shape4, Hq, T, qg, kc, kd, vc, vd, scale, out_sel, pos, sc, sws)
    out_sp = torch.empty_like(out)
    spws = dk.workspace(dk.decode_sparse_workspace_bytes(shape4, Hq, T, n_keep))
    dk.decode_attn_sparse(shape4, Hq, T, qg, kc, kd, vc, vd, pos, scale, out_sp, spws)
    torch.cuda.synchronize()
    out, out_sel, out_sp = (t.cpu().double().numpy() for t in (out, out_sel, out_sp))
    assert np.array_equal(out, out_sel)
    pos = pos.cpu().numpy()
    sc = sc.cpu().numpy()
    e_dense = e_sp = e_sc = 0.0
    for b in range(B):
        for h in range(H):
            kr, kl, ki = _oracle_cache(shape4, kc, b, h)
            vr, vl, vi = _oracle_cache(shape4, vc, b, h)
            qo = to_np(q[b, h * G:(h + 1) * G])
            ko, vo = oracle_mlp(kdw, dk.ACT_GELU), oracle_mlp(vdw, dk.ACT_GELU)
            e_dense = max(e_dense, rel_err_rows(out[b, h * G:(h + 1) * G],
                                                oracle.decode_head(qo, kr, kl, ki, ko, vr, vl, vi,
                                                                   vo, T, s, scale)))
            assert np.array_equal(pos[b, h], oracle.top_positions(sc[b, h], n_keep))
            _, mass = oracle.select_head(qo, kr, kl, ki, ko, T, s, scale, n_keep)
            e_sc = max(e_sc, check_selection(sc[b, h], pos[b, h], mass, n_keep,
                                             TOL[dk.BF16])[0])
            e_sp = max(e_sp, rel_err_rows(out_sp[b, h * G:(h + 1) * G],
                                          oracle.decode_head_sparse(qo, kr, kl, ki, ko, vr, vl, vi,
                                                                    vo, T, s, scale, pos[b, h])))
    say(f"[case] q4-decode {cfg}: dense {e_dense:.3e} sparse {e_sp:.3e} scores {e_sc:.3e}")
    assert max(e_dense, e_sp, e_sc) <= TOL[dk.BF16]
