"""CPU oracle for DeltaKV compression and decode attention (fp64, plain loops).

TEST INFRASTRUCTURE ONLY: this package is the checker the GPU path is compared
against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it; the product package never does, and the two share no code.

Method source: "DeltaKV: Residual-Based KV Cache Compression via Long-Range
Similarity" (gist.science summary), section 3 "Metodologia".  The arithmetic
lives in deltakv_oracle.c; this module only marshals numpy arrays to it and
strings the per-step functions together into per-head helpers.

Parity status per function (what pins it; the tests under tests/ hold them):
  build_refs        pinned: bit equality with the strided rows.
  select            pinned: brute force against numpy lexsort on tiny
                    integer inputs, crafted ties / duplicates / short prefixes.
  mlp / gelu        pinned: numpy matmul + scipy erf, standard-normal table
                    values, GELU limits.
  compress          pinned: closed form when all candidate refs are equal,
                    orthogonal identity pair round trip; latents under random
                    GELU weights equal numpy matmuls + scipy erf applied to
                    the numpy mean-and-residual of the listed references.
  reconstruct       pinned: orthogonal identity pair gives back the input;
                    under random GELU weights it equals the numpy rebuild.
  decode_head       pinned: with the identity pair it is dense attention over
                    the input rows; under random GELU weights it equals fp64
                    SDPA over rows rebuilt by numpy + scipy erf; with GELU
                    saturated off (each row KV_R + b2) or on (an affine
                    Decompressor) it equals SDPA over the closed-form rows.
  attention         pinned: torch scaled_dot_product_attention in fp64 and the
                    q = 0 closed form.
  reconstruct_at    pinned: orthogonal identity pair gives back the input rows
                    at the listed positions; rows equal the full rebuild's.
  decode_head_sparse pinned: the full position list gives the dense decode;
                    with the identity pair it is dense attention over x at the
                    listed positions; order, padding and duplicate invariants.
  group_attention_mass pinned: torch softmax weights summed over the group,
                    total mass = number of query rows.
  top_positions     pinned: a pure-Python sort on (-score, position) tuples,
                    crafted ties, n_keep >= T.
  decode_head_window pinned: the identity pair gives SDPA over the input rows
                    followed by the window rows; a window that repeats a row
                    weighs it twice; order-free in the window.
  quantize_latents  pinned: exact rational arithmetic (fractions.Fraction) on
                    random rows gives the same codes and scales; half-integer
                    quotients go to the even code; every value within half a
                    step of its code's value, row extremes on codes 0 and 15,
                    rows built from chosen codes recovered exactly, constant
                    rows exact.
  bf16_from_f64     pinned: exact rational rounding on random and near-midpoint
                    values; torch's fp32 -> bf16 rounding on fp32 inputs.
  reconstruction_loss pinned: zero for an orthogonal linear pair with d_c = d;
                    the oracle's own pinned MLP forward pass.
  reconstruction_grad pinned: central finite differences of
                    reconstruction_loss (which shares no code with it) on
                    every parameter of small GELU and identity pairs; zero
                    at the orthogonal pair; its loss equals
                    reconstruction_loss.
  gelu_vec / gelu_deriv pinned: the C oracle's gelu; finite differences.
  train_step        pinned: small steps lower the loss (descent direction);
                    the update is the stated rule on the pinned gradient.
  No page prints an intermediate value, so latents and decode outputs under
  random GELU weights are pinned by independent compositions (numpy, scipy,
  torch CPU) and closed forms, not by printed numbers.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

ACT_GELU = 0
ACT_IDENTITY = 1

_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_num_refs.restype = ctypes.c_int64
    lib.oracle_num_refs.argtypes = [ctypes.c_int64, ctypes.c_int32]
    lib.oracle_build_refs.restype = None
    lib.oracle_build_refs.argtypes = [_dp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _dp]
    lib.oracle_sq_dist.restype = ctypes.c_double
    lib.oracle_sq_dist.argtypes = [_dp, _dp, ctypes.c_int32]
    lib.oracle_select.restype = ctypes.c_int
    lib.oracle_select.argtypes = [_dp, _i64p, ctypes.c_int64, _dp, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p]
    lib.oracle_gelu.restype = ctypes.c_double
    lib.oracle_gelu.argtypes = [ctypes.c_double]
    lib.oracle_mlp.restype = None
    lib.oracle_mlp.argtypes = [_dp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_int32, _dp, _dp, _dp, _dp, ctypes.c_int32, _dp]
    lib.oracle_compress.restype = None
    lib.oracle_compress.argtypes = [_dp, ctypes.c_int64, ctypes.c_int32, _dp, _i32p,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    _dp, _dp, _dp, _dp, ctypes.c_int32, _dp, _dp, _dp]
    lib.oracle_reconstruct.restype = None
    lib.oracle_reconstruct.argtypes = [_dp, _dp, _i32p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, _dp, _dp, _dp, _dp, ctypes.c_int32, _dp]
    lib.oracle_reconstruct_at.restype = None
    lib.oracle_reconstruct_at.argtypes = [_dp, _dp, _i32p, _i64p, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, _dp, _dp, _dp, _dp,
                                          ctypes.c_int32, _dp]
    lib.oracle_group_attention_mass.restype = None
    lib.oracle_group_attention_mass.argtypes = [_dp, ctypes.c_int32, _dp, ctypes.c_int64,
                                                ctypes.c_int32, ctypes.c_double, _dp]
    lib.oracle_attention.restype = None
    lib.oracle_attention.argtypes = [_dp, ctypes.c_int32, _dp, _dp, ctypes.c_int64,
                                     ctypes.c_int32, ctypes.c_double, _dp]
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, typ=_dp):
    if a is None:
        return None
    return a.ctypes.data_as(typ)


@dataclass
class MLP:
    """One Linear -> act -> Linear block in fp64: w1 [hidden, in], b1 [hidden],
    w2 [out, hidden], b2 [out]; act is ACT_GELU or ACT_IDENTITY."""
    w1: np.ndarray
    b1: np.ndarray
    w2: np.ndarray
    b2: np.ndarray
    act: int = ACT_GELU

    def __post_init__(self):
        self.w1 = _f64(self.w1)
        self.w2 = _f64(self.w2)
        self.b1 = _f64(self.b1) if self.b1 is not None else np.zeros(self.w1.shape[0])
        self.b2 = _f64(self.b2) if self.b2 is not None else np.zeros(self.w2.shape[0])

    @property
    def din(self):
        return self.w1.shape[1]

    @property
    def hidden(self):
        return self.w1.shape[0]

    @property
    def dout(self):
        return self.w2.shape[0]


def num_refs(T: int, s: int) -> int:
    return int(_load().oracle_num_refs(int(T), int(s)))


def nonref_positions(T: int, s: int) -> np.ndarray:
    """Positions of the non-reference tokens among 0..T-1, increasing."""
    p = np.arange(T, dtype=np.int64)
    return p[p % s != 0]


def build_refs(x, s: int) -> np.ndarray:
    x = _f64(x)
    T, d = x.shape
    out = np.zeros((num_refs(T, s), d), dtype=np.float64)
    _load().oracle_build_refs(_ptr(x), T, d, s, _ptr(out))
    return out


def sq_dist(a, b) -> float:
    a = _f64(a)
    b = _f64(b)
    return float(_load().oracle_sq_dist(_ptr(a), _ptr(b), a.shape[0]))


def select(xt, pos, refs, s: int, k: int) -> np.ndarray:
    """Index rows (n, k) int32, -1 in unused slots."""
    xt = _f64(xt)
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64))
    refs = _f64(refs)
    n, d = xt.shape
    idx = np.full((n, k), -7, dtype=np.int32)
    rc = _load().oracle_select(_ptr(xt), _ptr(pos, _i64p), n, _ptr(refs), refs.shape[0],
                               d, s, k, _ptr(idx, _i32p))
    if rc != 0:
        raise ValueError(f"oracle_select failed with {rc}")
    return idx


def gelu(u: float) -> float:
    return float(_load().oracle_gelu(float(u)))


def mlp(inp, m: MLP) -> np.ndarray:
    inp = _f64(inp)
    n = inp.shape[0]
    out = np.zeros((n, m.dout), dtype=np.float64)
    _load().oracle_mlp(_ptr(inp), n, m.din, m.hidden, m.dout, _ptr(m.w1), _ptr(m.b1),
                       _ptr(m.w2), _ptr(m.b2), m.act, _ptr(out))
    return out


def compress(xt, refs, idx, m: MLP):
    """Returns (latent [n, d_c], kv_r [n, d], residual [n, d])."""
    xt = _f64(xt)
    refs = _f64(refs)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    n, d = xt.shape
    k = idx.shape[1]
    lat = np.zeros((n, m.dout), dtype=np.float64)
    kvr = np.zeros((n, d), dtype=np.float64)
    res = np.zeros((n, d), dtype=np.float64)
    _load().oracle_compress(_ptr(xt), n, d, _ptr(refs), _ptr(idx, _i32p), k, m.hidden,
                            m.dout, _ptr(m.w1), _ptr(m.b1), _ptr(m.w2), _ptr(m.b2), m.act,
                            _ptr(lat), _ptr(kvr), _ptr(res))
    return lat, kvr, res


def reconstruct(refs, latents, idx, T: int, s: int, m: MLP) -> np.ndarray:
    refs = _f64(refs)
    latents = _f64(latents)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    d = refs.shape[1]
    k = idx.shape[1]
    xhat = np.zeros((T, d), dtype=np.float64)
    _load().oracle_reconstruct(_ptr(refs), _ptr(latents), _ptr(idx, _i32p), T, s, d, k,
                               m.din, m.hidden, _ptr(m.w1), _ptr(m.b1), _ptr(m.w2),
                               _ptr(m.b2), m.act, _ptr(xhat))
    return xhat


def reconstruct_at(refs, latents, idx, positions, s: int, m: MLP) -> np.ndarray:
    """Rows of the given positions (each in [0, T)), rebuilt on demand."""
    refs = _f64(refs)
    latents = _f64(latents)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
    d = refs.shape[1]
    k = idx.shape[1]
    xhat = np.zeros((len(pos), d), dtype=np.float64)
    _load().oracle_reconstruct_at(_ptr(refs), _ptr(latents), _ptr(idx, _i32p),
                                  _ptr(pos, _i64p), len(pos), s, d, k, m.din, m.hidden,
                                  _ptr(m.w1), _ptr(m.b1), _ptr(m.w2), _ptr(m.b2), m.act,
                                  _ptr(xhat))
    return xhat


def attention(q, keys, vals, scale: float) -> np.ndarray:
    q = _f64(q)
    keys = _f64(keys)
    vals = _f64(vals)
    n_q, d = q.shape
    out = np.zeros((n_q, d), dtype=np.float64)
    _load().oracle_attention(_ptr(q), n_q, _ptr(keys), _ptr(vals), keys.shape[0], d,
                             float(scale), _ptr(out))
    return out


def group_attention_mass(q, keys, scale: float) -> np.ndarray:
    """sum over the query rows of each one's softmax attention weights [T]."""
    q = _f64(q)
    keys = _f64(keys)
    n_q, d = q.shape
    mass = np.zeros(keys.shape[0], dtype=np.float64)
    _load().oracle_group_attention_mass(_ptr(q), n_q, _ptr(keys), keys.shape[0], d,
                                        float(scale), _ptr(mass))
    return mass


def top_positions(scores, n_keep: int) -> np.ndarray:
    """The selection rule: the n_keep positions of largest score, equal scores
    ordered by the lower position, returned in increasing position order;
    with n_keep >= len(scores), every position and then -1 (int32)."""
    scores = np.asarray(scores)
    T = len(scores)
    if n_keep >= T:
        return np.concatenate([np.arange(T), np.full(n_keep - T, -1)]).astype(np.int32)
    order = np.lexsort((np.arange(T), -scores))   # primary: score descending
    return np.sort(order[:n_keep]).astype(np.int32)


def _bf16_round(x32):
    """fp32 -> the nearest bf16 value (ties to even), returned as fp32."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_from_f64(x):
    """fp64 values -> the nearest bf16 value, ties to the even significand,
    rounded once from the fp64 value (no passage through fp32), as fp64.
    A bf16 value carries 8 significant bits; below 2^-126 its step is 2^-133.
    Values that round past the largest finite bf16 become infinite."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # |x| in [2^(e-1), 2^e)
    step = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -step)), step)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)


def quantize_latents(z):
    """4-bit latent storage, one group per latent row (the 4-bit quantisation
    the DeltaKV page quotes its memory figure with; the format is this
    project's reading): rows z [n, d_c] of bf16 values (as any float array)
    -> codes [n, d_c] uint8 in 0..15, shift [n] and scale [n] (bf16 values as
    fp32).  Defined in IEEE fp64 arithmetic:
        shift = min of the row,
        scale = bf16(fl64(fl64(max - min) / 15)), rounded once from fp64,
        code  = clamp(rint(fl64(fl64(z - shift) / scale)), 0, 15),
    rint rounding half-integers to the even integer; a constant row has scale
    0 and codes 0."""
    z = np.asarray(z, dtype=np.float64)
    shift = z.min(axis=1)
    scale = bf16_from_f64((z.max(axis=1) - shift) / 15.0)
    safe = np.where(scale > 0, scale, 1.0)
    q = np.rint((z - shift[:, None]) / safe[:, None])
    codes = np.clip(q, 0, 15).astype(np.uint8)
    codes[scale == 0] = 0
    return codes, shift.astype(np.float32), scale.astype(np.float32)


def dequantize_latents(codes, shift, scale):
    """Latent rows from 4-bit storage: shift + code * scale (fp64, exact)."""
    return (np.asarray(shift, np.float64)[:, None]
            + np.asarray(codes, np.float64) * np.asarray(scale, np.float64)[:, None])


# ---- per-head helpers (composition of the steps above, no new arithmetic) ----

def compress_head(x, s: int, k: int, m: MLP, positions=None):
    """Offline compression of one head's rows x [T, d].

    Returns refs [ceil(T/s), d], idx [n, k] and latents [n, d_c] for the
    non-reference positions (all of them, or the given subset)."""
    x = _f64(x)
    T = x.shape[0]
    refs = build_refs(x, s)
    pos = nonref_positions(T, s) if positions is None else np.asarray(positions, np.int64)
    idx = select(x[pos], pos, refs, s, k)
    lat, _, _ = compress(x[pos], refs, idx, m)
    return refs, idx, lat


def decode_head(q_heads, k_refs, k_lat, k_idx, k_dec: MLP, v_refs, v_lat, v_idx,
                v_dec: MLP, T: int, s: int, scale: float) -> np.ndarray:
    """Attention of the query rows q_heads [G, d] (all mapped to this KV head)
    over the T tokens rebuilt from the compressed K and V of one head."""
    khat = reconstruct(k_refs, k_lat, k_idx, T, s, k_dec)
    vhat = reconstruct(v_refs, v_lat, v_idx, T, s, v_dec)
    return attention(q_heads, khat, vhat, scale)


def decode_head_sparse(q_heads, k_refs, k_lat, k_idx, k_dec: MLP, v_refs, v_lat, v_idx,
                       v_dec: MLP, T: int, s: int, scale: float, positions) -> np.ndarray:
    """Attention of q_heads [G, d] over only the listed positions of one head
    (on-demand reconstruction for a sparse selection).  Entries outside
    [0, T) are skipped; a position listed twice takes part twice; with no
    position left the output is zero."""
    pos = np.asarray(positions, dtype=np.int64).reshape(-1)
    pos = pos[(pos >= 0) & (pos < T)]
    q_heads = _f64(q_heads)
    if len(pos) == 0:
        return np.zeros_like(q_heads)
    khat = reconstruct_at(k_refs, k_lat, k_idx, pos, s, k_dec)
    vhat = reconstruct_at(v_refs, v_lat, v_idx, pos, s, v_dec)
    return attention(q_heads, khat, vhat, scale)


def select_head(q_heads, k_refs, k_lat, k_idx, k_dec: MLP, T: int, s: int, scale: float,
                n_keep: int):
    """Query-aware selection for one KV head: the attention mass of every
    position (rebuilt keys, summed over the query rows q_heads [G, d]) and the
    positions the selection rule keeps.  Returns (positions, mass)."""
    khat = reconstruct(k_refs, k_lat, k_idx, T, s, k_dec)
    mass = group_attention_mass(q_heads, khat, scale)
    return top_positions(mass, n_keep), mass


def decode_head_window(q_heads, k_refs, k_lat, k_idx, k_dec: MLP, v_refs, v_lat, v_idx,
                       v_dec: MLP, T: int, s: int, scale: float, k_win, v_win) -> np.ndarray:
    """Attention of q_heads [G, d] over the T rebuilt tokens of one head plus
    n_win exact rows (k_win, v_win [n_win, d]: a recent window not yet
    compressed, or attention sinks kept verbatim)."""
    khat = reconstruct(k_refs, k_lat, k_idx, T, s, k_dec)
    vhat = reconstruct(v_refs, v_lat, v_idx, T, s, v_dec)
    keys = np.concatenate([khat, _f64(k_win)], axis=0)
    vals = np.concatenate([vhat, _f64(v_win)], axis=0)
    return attention(q_heads, keys, vals, scale)



# ---------------------------------------------------------------- training (MSE)
# DeltaKV page, section 3, "Obiettivo di Training Ibrido": the Compressor and
# Decompressor are trained with a reconstruction-fidelity (MSE) term next to a
# next-token term.  Only the MSE term is defined without a language model:
# for residual rows D [n, d], the loss is the mean over the n x d entries of
# (decompressor(compressor(D)) - D)^2, which is the mean squared error of the
# rebuilt rows KV_R + decompressor(latent) against the input rows.  The pages
# name no optimiser; the plainest reading is gradient descent, here with an
# optional heavy-ball momentum: v <- mu v + g, w <- w - lr v (mu = 0: plain).

def _erf_vec(u):
    from scipy.special import erf
    return erf(u)


def gelu_vec(u):
    """GELU, erf form, elementwise in fp64."""
    u = _f64(u)
    return 0.5 * u * (1.0 + _erf_vec(u / np.sqrt(2.0)))


def gelu_deriv(u):
    """d GELU / du = Phi(u) + u phi(u) (Phi, phi: the standard normal cdf and
    density), elementwise in fp64."""
    u = _f64(u)
    return 0.5 * (1.0 + _erf_vec(u / np.sqrt(2.0))) + u * np.exp(-0.5 * u * u) / np.sqrt(2.0 * np.pi)


def reconstruction_loss(delta, comp: MLP, dec: MLP) -> float:
    """The MSE term: mean over all entries of (dec(comp(delta)) - delta)^2,
    with the forward pass of the oracle's MLP."""
    delta = _f64(delta)
    y = mlp(mlp(delta, comp), dec)
    return float(np.mean((y - delta) ** 2))


def pack_params(comp: MLP, dec: MLP) -> np.ndarray:
    """W1c, b1c, W2c, b2c, W1d, b1d, W2d, b2d, each row-major, concatenated."""
    return np.concatenate([a.reshape(-1) for a in (comp.w1, comp.b1, comp.w2, comp.b2,
                                                   dec.w1, dec.b1, dec.w2, dec.b2)])


def unpack_params(vec, comp: MLP, dec: MLP):
    """New (comp, dec) with the shapes and activations of comp, dec and the
    values of vec (the order of pack_params)."""
    vec = _f64(vec)
    shapes = [a.shape for a in (comp.w1, comp.b1, comp.w2, comp.b2, dec.w1, dec.b1, dec.w2,
                                dec.b2)]
    parts, o = [], 0
    for sh in shapes:
        n = int(np.prod(sh))
        parts.append(vec[o:o + n].reshape(sh))
        o += n
    assert o == len(vec)
    return (MLP(parts[0], parts[1], parts[2], parts[3], comp.act),
            MLP(parts[4], parts[5], parts[6], parts[7], dec.act))


def reconstruction_grad(delta, comp: MLP, dec: MLP):
    """(loss, packed gradient) of the MSE term by backpropagation through the
    two blocks: each layer u = a W^T + b passes dL/du back as dL/da =
    (dL/du) W and contributes dL/dW = (dL/du)^T a, dL/db = sum over rows of
    dL/du; an activation passes dL/dphi times phi'(u)."""
    D = _f64(delta)
    n, d = D.shape
    phi = lambda u, act: gelu_vec(u) if act == ACT_GELU else u
    dphi = lambda u, act: gelu_deriv(u) if act == ACT_GELU else np.ones_like(u)
    a1 = D @ comp.w1.T + comp.b1
    h1 = phi(a1, comp.act)
    z = h1 @ comp.w2.T + comp.b2
    a2 = z @ dec.w1.T + dec.b1
    h2 = phi(a2, dec.act)
    y = h2 @ dec.w2.T + dec.b2
    e = y - D
    loss = float(np.mean(e * e))
    gy = 2.0 * e / (n * d)
    g_w2d, g_b2d = gy.T @ h2, gy.sum(axis=0)
    ga2 = (gy @ dec.w2) * dphi(a2, dec.act)
    g_w1d, g_b1d = ga2.T @ z, ga2.sum(axis=0)
    gz = ga2 @ dec.w1
    g_w2c, g_b2c = gz.T @ h1, gz.sum(axis=0)
    ga1 = (gz @ comp.w2) * dphi(a1, comp.act)
    g_w1c, g_b1c = ga1.T @ D, ga1.sum(axis=0)
    grad = np.concatenate([a.reshape(-1) for a in (g_w1c, g_b1c, g_w2c, g_b2c, g_w1d, g_b1d,
                                                   g_w2d, g_b2d)])
    return loss, grad


def train_step(delta, comp: MLP, dec: MLP, lr: float, momentum: float = 0.0, velocity=None):
    """One step: (loss before the step, gradient, new comp, new dec, new
    velocity)."""
    loss, g = reconstruction_grad(delta, comp, dec)
    v = g if velocity is None else momentum * _f64(velocity) + g
    new = pack_params(comp, dec) - lr * v
    c2, d2 = unpack_params(new, comp, dec)
    return loss, g, c2, d2, v
