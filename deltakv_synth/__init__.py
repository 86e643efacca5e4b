"""Seeded synthetic inputs for DeltaKV compression and decode attention.

This module only draws random inputs (KV rows, MLP weights, queries) and holds
the workload shapes.  It contains none of the method's arithmetic, so both the
GPU path's tests/benchmark and the CPU oracle can take their inputs from it.

KV rows follow the two observations of "DeltaKV: Residual-Based KV Cache
Compression via Long-Range Similarity", section 2: a few shared high-norm
directions dominate every row (anisotropy), and rows that are close to one
another recur at positions far apart (each row joins one of C clusters chosen
uniformly at random per position).  A row is

    x_t = sum_m c_{t,m} * (dir_norm * u_m) + centroid_scale * mu_{a(t)} + eps_t

with u_m, mu_c unit vectors drawn from N(0, I) and normalised, c_{t,m} ~ N(0,1),
a(t) ~ U{0..C-1}, eps_t ~ N(0, noise_std^2 I), then rounded (RNE) to the
storage dtype.  Every unit (sequence, layer, KV head, stream) is an
independent draw keyed by a tuple of integers.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch

# purposes, used as the last element of a seed key
P_DIRS, P_CENTROIDS, P_COEFFS, P_ASSIGN, P_NOISE, P_WEIGHTS, P_QUERIES, P_BIAS, P_SELECT = range(9)


def seed_of(*key: int) -> int:
    """63-bit seed from an integer tuple via numpy's SeedSequence."""
    st = np.random.SeedSequence([int(v) for v in key]).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _gen(device, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*key))
    return g


def kv_rows(T: int, d: int, n_dirs: int, n_centroids: int, key: Tuple[int, ...],
            dtype=torch.float32, device="cpu", dir_norm: float = 20.0,
            centroid_scale: float = 5.0, noise_std: float = 0.1,
            t0: int = 0) -> torch.Tensor:
    """Rows t0..t0+T-1 of one unit's K or V stream, shape [T, d].

    The directions and centroids depend only on `key`; the per-row draws are
    made in blocks of 4096 positions keyed by the block number, so a row's
    value does not depend on how the rows are requested (t0, T)."""
    f32 = torch.float32
    u = torch.randn(n_dirs, d, generator=_gen(device, *key, P_DIRS), device=device, dtype=f32)
    u = u / u.norm(dim=1, keepdim=True)
    mu = torch.randn(n_centroids, d, generator=_gen(device, *key, P_CENTROIDS), device=device,
                     dtype=f32)
    mu = mu / mu.norm(dim=1, keepdim=True)
    blk = 4096
    out = torch.empty(T, d, device=device, dtype=dtype)
    b0, b1 = t0 // blk, (t0 + T - 1) // blk if T > 0 else t0 // blk - 1
    for b in range(b0, b1 + 1):
        c = torch.randn(blk, n_dirs, generator=_gen(device, *key, P_COEFFS, b), device=device,
                        dtype=f32)
        a = torch.randint(0, n_centroids, (blk,), generator=_gen(device, *key, P_ASSIGN, b),
                          device=device)
        e = torch.randn(blk, d, generator=_gen(device, *key, P_NOISE, b), device=device, dtype=f32)
        rows = (c @ (dir_norm * u)) + centroid_scale * mu[a] + noise_std * e
        lo = max(t0, b * blk)
        hi = min(t0 + T, (b + 1) * blk)
        out[lo - t0:hi - t0] = rows[lo - b * blk:hi - b * blk].to(dtype)
    return out


def xavier_mlp(din: int, hidden: int, dout: int, key: Tuple[int, ...], dtype=torch.float32,
               device="cpu", bias_std: float = 0.0) -> dict:
    """Linear(din->hidden) -> act -> Linear(hidden->dout) weights, Xavier-uniform
    (bound sqrt(6/(fan_in+fan_out))), row-major [out, in] in `dtype`; biases
    fp32, zero unless bias_std > 0 (then N(0, bias_std^2))."""
    g = _gen(device, *key, P_WEIGHTS)
    lim1 = (6.0 / (din + hidden)) ** 0.5
    lim2 = (6.0 / (hidden + dout)) ** 0.5
    w1 = (torch.rand(hidden, din, generator=g, device=device) * 2 - 1) * lim1
    w2 = (torch.rand(dout, hidden, generator=g, device=device) * 2 - 1) * lim2
    if bias_std > 0:
        gb = _gen(device, *key, P_BIAS)
        b1 = torch.randn(hidden, generator=gb, device=device) * bias_std
        b2 = torch.randn(dout, generator=gb, device=device) * bias_std
    else:
        b1 = torch.zeros(hidden, device=device)
        b2 = torch.zeros(dout, device=device)
    return {"w1": w1.to(dtype).contiguous(), "b1": b1.float().contiguous(),
            "w2": w2.to(dtype).contiguous(), "b2": b2.float().contiguous()}


def queries(n: int, d: int, key: Tuple[int, ...], dtype=torch.float32,
            device="cpu") -> torch.Tensor:
    """n query rows ~ N(0, I), shape [n, d]."""
    g = _gen(device, *key, P_QUERIES)
    return torch.randn(n, d, generator=g, device=device).to(dtype)


def selections(n_lists: int, T: int, n_sel: int, key: Tuple[int, ...],
               device="cpu") -> torch.Tensor:
    """n_lists position lists, each n_sel distinct positions drawn uniformly
    from [0, T) and sorted ascending: int32 [n_lists, n_sel].  A stand-in for
    a sparse-attention selector's output (which positions a query-aware
    selector keeps depends on a trained model; only the list sizes matter to
    the cost of rebuilding them)."""
    g = _gen(device, *key, P_SELECT)
    out = torch.empty(n_lists, n_sel, dtype=torch.int32, device=device)
    for i in range(n_lists):
        out[i] = torch.randperm(T, generator=g, device=device)[:n_sel].sort().values
    return out


@dataclass(frozen=True)
class Workload:
    """Shapes and generator settings of one synthetic workload."""
    name: str
    layers: int
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    T: int
    stride: int
    k: int
    d_c: int
    hidden: int
    dtype: str            # "fp32" or "bf16"
    n_dirs: int
    n_centroids: int
    decode_steps: int
    chunk: Optional[int] = None   # streaming: prompt compressed in chunks of this size
    appends: int = 0              # streaming: tokens appended during decode

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


# The five workloads, named by what they are.  Shapes: Llama-3.1-8B K/V heads
# (8 KV heads, 32 query heads, head_dim 128, 32 layers) at up to 128k context.
WORKLOADS = {
    "tiny-1head-T512-fp32": Workload(
        "tiny-1head-T512-fp32", layers=1, batch=1, kv_heads=1, q_heads=1, head_dim=64,
        T=512, stride=16, k=4, d_c=16, hidden=128, dtype="fp32", n_dirs=4, n_centroids=32,
        decode_steps=1),
    "llama8b-1layer-T32k-bf16": Workload(
        "llama8b-1layer-T32k-bf16", layers=1, batch=1, kv_heads=8, q_heads=32, head_dim=128,
        T=32768, stride=16, k=4, d_c=32, hidden=256, dtype="bf16", n_dirs=8,
        n_centroids=1024, decode_steps=256),
    "llama8b-32layer-T128k-bf16": Workload(
        "llama8b-32layer-T128k-bf16", layers=32, batch=1, kv_heads=8, q_heads=32,
        head_dim=128, T=131072, stride=16, k=4, d_c=32, hidden=256, dtype="bf16", n_dirs=8,
        n_centroids=1024, decode_steps=128),
    "llama8b-32layer-T128k-batch8-bf16": Workload(
        "llama8b-32layer-T128k-batch8-bf16", layers=32, batch=8, kv_heads=8, q_heads=32,
        head_dim=128, T=131072, stride=16, k=4, d_c=32, hidden=256, dtype="bf16", n_dirs=8,
        n_centroids=1024, decode_steps=128),
    "llama8b-32layer-T128k-stream-s8k8-bf16": Workload(
        "llama8b-32layer-T128k-stream-s8k8-bf16", layers=32, batch=1, kv_heads=8,
        q_heads=32, head_dim=128, T=131072, stride=8, k=8, d_c=16, hidden=256, dtype="bf16",
        n_dirs=8, n_centroids=1024, decode_steps=1024, chunk=4096, appends=1024),
}


def unit_key(workload_index: int, b: int, layer: int, head: int, stream: int) -> Tuple[int, ...]:
    """Seed key of one unit; stream 0 = K, 1 = V."""
    return (0, workload_index, b, layer, head, stream)


def workload_index(name: str) -> int:
    return list(WORKLOADS).index(name)
