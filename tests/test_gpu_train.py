"""GPU parity of the residual rows and of the Compressor / Decompressor MSE
training step (DeltaKV page, section 3: the residual of "Processo di
Compressione" and the MSE term of "Obiettivo di Training Ibrido").

  - residuals: against the oracle's residual rows (fp64 mean of the same
    reference rows) on the GPU's own stored idx; fp32 bar 1e-4;
  - one step: loss, gradient (each layer's weights and bias), updated
    weights and velocity against the oracle's fp64 step on the same rows and
    weights; fp32 bar 1e-4 relative to each layer array's largest entry; the bf16 copies are the round-to-
    nearest-even bf16 of the GPU's updated fp32 weights, bit for bit;
  - many steps: the GPU's loss curve follows the oracle's, and training on
    residual rows of the synthetic generator lowers the reconstruction error.
"""
import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
import oracle
from parity import gpu_compress, gpu_mlp, idx_to_oracle, make_kv, make_mlp, rel_err_rows, say, \
    to_np

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4


def _residual_case(name, B, H, T, d, s, k, dc, hid, dtype, t0, t1, seed):
    say(f"[case] {name}: B={B} H={H} T={T} d={d} s={s} k={k} dtype={dtype} [{t0}, {t1})")
    tdt = torch.float32 if dtype == dk.F32 else torch.bfloat16
    shape = dk.Shape(B, H, d, s, k, dc, T, dtype)
    x = make_kv(B, H, T, d, tdt, key=(seed, 0))
    cw, _ = make_mlp(d, hid, dc, tdt, key=(seed, 1))
    cache = gpu_compress(shape, x, gpu_mlp(cw, dk.ACT_GELU))
    pos = oracle.nonref_positions(t1, s)
    pos = pos[pos >= t0]
    out = torch.full((B, H, len(pos), d), float("nan"), device="cuda")
    xs = x[:, :, t0:t1].contiguous().cuda()
    dk.residuals(shape, xs, t0, t1, cache, out if len(pos) else None)
    torch.cuda.synchronize()
    if len(pos) == 0:
        return None
    got = out.cpu().double().numpy()
    err = 0.0
    R = oracle.num_refs(T, s)
    for b in range(B):
        for h in range(H):
            refs = to_np(cache.refs[b, h, :R].cpu())
            qord = (pos // s) * (s - 1) + (pos % s) - 1
            idx = idx_to_oracle(cache.idx[b, h].cpu()[torch.from_numpy(qord)])
            _, _, res = oracle.compress(to_np(x[b, h])[pos], refs, idx,
                                        oracle.MLP(np.zeros((1, d)), None, np.zeros((dc, 1)),
                                                   None))
            err = max(err, rel_err_rows(got[b, h], res))
    say(f"[case] {name}: residual rel err {err:.3e}")
    assert err <= F32_TOL
    return got


def test_residuals_bf16_cache():
    _residual_case("residuals-bf16", 1, 2, 700, 128, 16, 4, 32, 256, dk.BF16, 0, 700, seed=601)


def test_residuals_fp32_subrange_k8():
    # a sub-range [t0, t1) that starts and ends mid-stride, fp32 storage, k = 8
    _residual_case("residuals-fp32", 2, 1, 500, 64, 8, 8, 16, 128, dk.F32, 133, 411, seed=602)


def test_residuals_of_reference_positions_only_write_nothing():
    _residual_case("residuals-refs-only", 1, 1, 300, 64, 16, 4, 16, 128, dk.BF16, 32, 33,
                   seed=603)


def _pair(d, h, dc, act, seed, scale=0.5):
    rng = np.random.default_rng(seed)
    fan = lambda a, b: scale * np.sqrt(2.0 / (a + b))
    comp = oracle.MLP(rng.normal(0, fan(d, h), (h, d)), rng.normal(0, 0.05, h),
                      rng.normal(0, fan(h, dc), (dc, h)), rng.normal(0, 0.05, dc), act)
    dec = oracle.MLP(rng.normal(0, fan(dc, h), (h, dc)), rng.normal(0, 0.05, h),
                     rng.normal(0, fan(h, d), (d, h)), rng.normal(0, 0.05, d), act)
    # fp32 values both sides start from
    for m in (comp, dec):
        for a in ("w1", "b1", "w2", "b2"):
            setattr(m, a, getattr(m, a).astype(np.float32).astype(np.float64))
    return comp, dec


def _gpu_f32(m):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return dk.MlpF32(t(m.w1), t(m.b1), t(m.w2), t(m.b2), m.act)


def _rel_block(a, b):
    """Largest entry error of a layer's array relative to its largest entry
    (rows can be small by cancellation, e.g. one row's outer product, where a
    per-row ratio measures that cancellation rather than the product)."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-30))


def _blocks(vec, comp, dec):
    c, d = oracle.unpack_params(vec, comp, dec)
    return [("W1c", c.w1), ("b1c", c.b1[None]), ("W2c", c.w2), ("b2c", c.b2[None]),
            ("W1d", d.w1), ("b1d", d.b1[None]), ("W2d", d.w2), ("b2d", d.b2[None])]


@pytest.mark.parametrize("cfg", [
    # (n, d, h, dc, act, momentum)
    (1000, 128, 256, 32, dk.ACT_GELU, 0.9),     # the Llama-shaped pair, ragged row count
    (64, 64, 128, 16, dk.ACT_GELU, 0.0),        # one row tile, plain descent
    (1, 128, 256, 16, dk.ACT_IDENTITY, 0.5),    # a single row
    (777, 64, 100, 24, dk.ACT_GELU, 0.0),       # widths off the 64-wide tiles
], ids=["llama-1000", "tile-64", "one-row", "ragged-widths"])
def test_train_step_matches_the_oracle(cfg):
    n, d, h, dc, act, mom = cfg
    say(f"[case] train-step n={n} d={d} h={h} dc={dc} act={act} momentum={mom}")
    comp, dec = _pair(d, h, dc, act, seed=610 + n)
    rng = np.random.default_rng(620 + n)
    delta = rng.normal(0, 1.0, (n, d)).astype(np.float32).astype(np.float64)
    npar = len(oracle.pack_params(comp, dec))
    vel0 = rng.normal(0, 0.01, npar).astype(np.float32).astype(np.float64)
    lr = 0.05
    loss_o, g_o, c_o, d_o, v_o = oracle.train_step(delta, comp, dec, lr, mom,
                                                    vel0 if mom else None)
    gc, gd = _gpu_f32(comp), _gpu_f32(dec)
    wsb, npar_g = dk.train_workspace_bytes(gc, gd, n)
    assert npar_g == npar
    ws = dk.workspace(wsb)
    ws.fill_(0xFF)
    vel = torch.from_numpy(vel0.astype(np.float32)).cuda() if mom else None
    loss = torch.full((1,), float("nan"), device="cuda")
    grad = torch.full((npar,), float("nan"), device="cuda")
    bw = [torch.empty(m.shape, dtype=torch.bfloat16, device="cuda")
          for m in (comp.w1, comp.w2, dec.w1, dec.w2)]
    dk.train_step(torch.from_numpy(delta.astype(np.float32)).cuda(), gc, gd, lr, ws, mom, vel,
                  loss, grad, bw)
    torch.cuda.synchronize()
    lg = float(loss.item())
    assert abs(lg - loss_o) <= F32_TOL * loss_o, (lg, loss_o)
    g_g = grad.cpu().double().numpy()
    worst = 0.0
    for (nm, a), (_, b) in zip(_blocks(g_g, comp, dec), _blocks(g_o, comp, dec)):
        e = _rel_block(a, b)
        worst = max(worst, e)
        assert e <= F32_TOL, f"gradient of {nm}: rel err {e:.3e}"
    new_g = np.concatenate([t.cpu().double().numpy().reshape(-1)
                            for t in (gc.w1, gc.b1, gc.w2, gc.b2, gd.w1, gd.b1, gd.w2, gd.b2)])
    new_o = oracle.pack_params(c_o, d_o)
    for (nm, a), (_, b) in zip(_blocks(new_g, comp, dec), _blocks(new_o, comp, dec)):
        assert _rel_block(a, b) <= F32_TOL, f"updated {nm}"
    if mom:
        v_g = vel.cpu().double().numpy()
        for (nm, a), (_, b) in zip(_blocks(v_g, comp, dec), _blocks(v_o, comp, dec)):
            assert _rel_block(a, b) <= F32_TOL, f"velocity of {nm}"
    # bf16 copies: the round-to-nearest-even bf16 of the GPU's own new weights
    for t, w in zip(bw, (gc.w1, gc.w2, gd.w1, gd.w2)):
        want = oracle.bf16_from_f64(w.cpu().double().numpy())
        assert np.array_equal(t.cpu().double().numpy(), want)
    say(f"[case] train-step n={n}: loss rel err {abs(lg - loss_o) / loss_o:.2e}, "
        f"gradient rel err {worst:.2e}")


def test_training_on_synthetic_residuals_lowers_the_reconstruction_error():
    # residual rows of a compressed Llama-shaped layer (both K heads of a
    # small cache), 60 steps on the GPU next to 60 oracle steps from the same
    # start: the curves agree and the error falls
    B, H, T, d, s, k, dc, hid = 1, 2, 1200, 128, 16, 4, 32, 256
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    x = make_kv(B, H, T, d, torch.bfloat16, key=(630, 0))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(630, 1))
    cache = gpu_compress(shape, x, gpu_mlp(cw, dk.ACT_GELU))
    n_per = T - oracle.num_refs(T, s)
    res = torch.empty(B, H, n_per, d, device="cuda")
    dk.residuals(shape, x.cuda(), 0, T, cache, res)
    delta = res.reshape(-1, d).contiguous()
    comp, dec = _pair(d, hid, dc, dk.ACT_GELU, seed=631, scale=0.3)
    gc, gd = _gpu_f32(comp), _gpu_f32(dec)
    n = delta.shape[0]
    ws = dk.workspace(dk.train_workspace_bytes(gc, gd, n)[0])
    npar = len(oracle.pack_params(comp, dec))
    vel = torch.zeros(npar, device="cuda")
    loss = torch.zeros(1, device="cuda")
    d_np = delta.cpu().double().numpy()
    v_o = np.zeros(npar)
    lr, mom, steps = 0.1, 0.9, 60
    curve_g, curve_o = [], []
    for _ in range(steps):
        dk.train_step(delta, gc, gd, lr, ws, mom, vel, loss)
        curve_g.append(float(loss.item()))
        lo, _, comp, dec, v_o = oracle.train_step(d_np, comp, dec, lr, mom, v_o)
        curve_o.append(lo)
    torch.cuda.synchronize()
    rel = max(abs(a - b) / b for a, b in zip(curve_g, curve_o))
    say(f"[case] train-60: loss {curve_o[0]:.4f} -> {curve_o[-1]:.4f} (oracle), "
        f"largest relative gap of the GPU curve {rel:.2e}")
    assert rel <= 1e-3
    assert curve_g[-1] < 0.3 * curve_g[0]
