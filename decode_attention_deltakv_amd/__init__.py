"""Python binding of libdeltakv.so: DeltaKV compression and decode attention
on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
libdeltakv.so, reached through its C ABI (include/deltakv.h); torch provides
device memory and the current stream.  There is no fallback: if the library
is missing, loading this package's functions raises.

The functions keep the C names (without the `deltakv_` prefix, which is also
available as an alias):

    cache_bytes(shape)                         -> dict of byte sizes
    compress_workspace_bytes(shape, t0, t1)    -> int
    decode_workspace_bytes(shape, Hq, T)       -> int
    build_refs(shape, x, t0, t1, cache)
    compress(shape, x, t0, t1, compressor, cache, workspace, stats=None)
    decode_attn(shape, Hq, T, q, k_cache, k_dec, v_cache, v_dec, scale, out, workspace)
    decode_attn_noalloc(shape, Hq, T, q, k_cache, k_dec, v_cache, v_dec, scale, out)
    decode_sparse_workspace_bytes(shape, Hq, T, n_sel) -> int
    decode_attn_sparse(shape, Hq, T, q, k_cache, k_dec, v_cache, v_dec, positions, scale,
                       out, workspace)
    decode_select_workspace_bytes(shape, Hq, T) -> int
    decode_window_workspace_bytes(shape, Hq, T, n_win) -> int
    decode_varlen_workspace_bytes(shape, Hq, max_T) -> int
    decode_attn_varlen(shape, Hq, lengths, max_tokens, q, k_cache, k_dec, v_cache, v_dec,
                       scale, out, workspace)
    decode_attn_window(shape, Hq, T, q, k_cache, k_dec, v_cache, v_dec, k_win, v_win, scale,
                       out, workspace)
    decode_attn_select(shape, Hq, T, q, k_cache, k_dec, v_cache, v_dec, scale, out,
                       positions, scores, workspace)

`Cache` and `Mlp` below only hold torch tensors and build the C structs.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdeltakv.so")

F32, BF16 = 0, 1
ACT_GELU, ACT_IDENTITY = 0, 1
LATENT_DTYPE, LATENT_Q4 = 0, 1

STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "CAPACITY", 4: "WORKSPACE",
                5: "HIP"}


class DeltaKVError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"deltakv: {STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class CShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("stride", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_c", ctypes.c_int32), ("capacity", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("latent_format", ctypes.c_int32),
                ("page_refs", ctypes.c_int32)]


class CMlp(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("in_dim", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("out_dim", ctypes.c_int32), ("act", ctypes.c_int32)]


class CCache(ctypes.Structure):
    _fields_ = [("refs", ctypes.c_void_p), ("ref_sqnorm", ctypes.c_void_p),
                ("latents", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("n_built", ctypes.c_int64), ("n_compressed", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("n_pages", ctypes.c_int64)]


class CMlpF32(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b2", ctypes.c_void_p), ("in_dim", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("out_dim", ctypes.c_int32), ("act", ctypes.c_int32)]


class CAppendItem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("cache", ctypes.POINTER(CCache)),
                ("compressor", ctypes.POINTER(CMlp))]


_lib = None
_SZ = ctypes.c_size_t
_P = ctypes.c_void_p


def lib():
    """The loaded libdeltakv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m decode_attention_deltakv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    sp = ctypes.POINTER(CShape)
    L.deltakv_cache_bytes.argtypes = [sp, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ),
                                      ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]
    L.deltakv_page_bytes.argtypes = [sp, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ),
                                     ctypes.POINTER(_SZ), ctypes.POINTER(_SZ),
                                     ctypes.POINTER(ctypes.c_int32)]
    L.deltakv_compress_workspace_bytes.argtypes = [sp, ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.POINTER(_SZ)]
    L.deltakv_decode_workspace_bytes.argtypes = [sp, ctypes.c_int32, ctypes.c_int64,
                                                 ctypes.POINTER(_SZ)]
    L.deltakv_build_refs.argtypes = [sp, _P, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.POINTER(CCache), _P]
    L.deltakv_compress.argtypes = [sp, _P, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(CMlp),
                                   ctypes.POINTER(CCache), _P, _SZ, _P, _P]
    L.deltakv_decode_attn.argtypes = [sp, ctypes.c_int32, ctypes.c_int64, _P,
                                      ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                      ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                      ctypes.c_float, _P, _P, _SZ, _P]
    L.deltakv_decode_attn_noalloc.argtypes = [sp, ctypes.c_int32, ctypes.c_int64, _P,
                                              ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                              ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                              ctypes.c_float, _P, _P]
    L.deltakv_decode_sparse_workspace_bytes.argtypes = [sp, ctypes.c_int32, ctypes.c_int64,
                                                        ctypes.c_int32, ctypes.POINTER(_SZ)]
    L.deltakv_decode_attn_sparse.argtypes = [sp, ctypes.c_int32, ctypes.c_int64, _P,
                                             ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                             ctypes.POINTER(CCache), ctypes.POINTER(CMlp), _P,
                                             ctypes.c_int32, ctypes.c_float, _P, _P, _SZ, _P]
    L.deltakv_decode_select_workspace_bytes.argtypes = [sp, ctypes.c_int32, ctypes.c_int64,
                                                        ctypes.POINTER(_SZ)]
    L.deltakv_decode_attn_select.argtypes = [sp, ctypes.c_int32, ctypes.c_int64, _P,
                                             ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                             ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                             ctypes.c_float, _P, ctypes.c_int32, _P, _P, _P, _SZ,
                                             _P]
    L.deltakv_decode_window_workspace_bytes.argtypes = [sp, ctypes.c_int32, ctypes.c_int64,
                                                        ctypes.c_int64, ctypes.POINTER(_SZ)]
    L.deltakv_decode_attn_window.argtypes = [sp, ctypes.c_int32, ctypes.c_int64, _P,
                                             ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                             ctypes.POINTER(CCache), ctypes.POINTER(CMlp), _P,
                                             _P, ctypes.c_int64, ctypes.c_float, _P, _P, _SZ, _P]
    L.deltakv_decode_varlen_workspace_bytes.argtypes = [sp, ctypes.c_int32, ctypes.c_int64,
                                                        ctypes.POINTER(_SZ)]
    L.deltakv_decode_attn_varlen.argtypes = [sp, ctypes.c_int32, _P, ctypes.c_int64,
                                             _P, ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                             ctypes.POINTER(CCache), ctypes.POINTER(CMlp),
                                             ctypes.c_float, _P, _P, _SZ, _P]
    L.deltakv_append_workspace_bytes.argtypes = [sp, ctypes.c_int64, ctypes.c_int32,
                                                 ctypes.POINTER(_SZ)]
    L.deltakv_append.argtypes = [sp, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.POINTER(CAppendItem), _P, _SZ, _P]
    L.deltakv_residuals.argtypes = [sp, _P, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.POINTER(CCache), _P, _P]
    L.deltakv_train_workspace_bytes.argtypes = [ctypes.POINTER(CMlpF32), ctypes.POINTER(CMlpF32),
                                                ctypes.c_int64, ctypes.POINTER(_SZ),
                                                ctypes.POINTER(ctypes.c_int64)]
    L.deltakv_train_step.argtypes = [ctypes.c_int64, _P, ctypes.POINTER(CMlpF32),
                                     ctypes.POINTER(CMlpF32), ctypes.c_float, ctypes.c_float,
                                     _P, _P, _P, ctypes.POINTER(_P), _P, _SZ, _P]
    for name in ("deltakv_residuals", "deltakv_train_workspace_bytes", "deltakv_train_step",
                 "deltakv_append_workspace_bytes", "deltakv_append",
                 "deltakv_cache_bytes", "deltakv_page_bytes", "deltakv_compress_workspace_bytes",
                 "deltakv_decode_workspace_bytes", "deltakv_build_refs", "deltakv_compress",
                 "deltakv_decode_attn", "deltakv_decode_sparse_workspace_bytes",
                 "deltakv_decode_attn_sparse", "deltakv_decode_select_workspace_bytes",
                 "deltakv_decode_attn_select", "deltakv_decode_window_workspace_bytes",
                 "deltakv_decode_attn_window", "deltakv_decode_varlen_workspace_bytes",
                 "deltakv_decode_attn_varlen", "deltakv_decode_attn_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    L.deltakv_peak_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]
    L.deltakv_peak_probe.restype = ctypes.c_int
    L.deltakv_status_string.argtypes = [ctypes.c_int]
    L.deltakv_status_string.restype = ctypes.c_char_p
    L.deltakv_last_error.argtypes = []
    L.deltakv_last_error.restype = ctypes.c_char_p
    L.deltakv_version.argtypes = []
    L.deltakv_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise DeltaKVError(status, lib().deltakv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libdeltakv must be contiguous")
    return t.data_ptr()


def _stream():
    # torch's current HIP stream; without a visible device only the argument
    # checks of the library can run, and they never touch the stream
    if not torch.cuda.is_available():
        return None
    return torch.cuda.current_stream().cuda_stream


@dataclass(frozen=True)
class Shape:
    batch: int
    num_kv_heads: int
    head_dim: int
    stride: int
    k: int
    d_c: int
    capacity: int
    dtype: int = BF16
    latent_format: int = 0   # LATENT_DTYPE or LATENT_Q4
    page_refs: int = 0       # 0: unit-contiguous arrays; else reference rows per page

    def c(self) -> CShape:
        return CShape(self.batch, self.num_kv_heads, self.head_dim, self.stride, self.k,
                      self.d_c, self.capacity, self.dtype, self.latent_format, self.page_refs)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == F32 else torch.bfloat16

    @property
    def n_refs(self):
        return -(-self.capacity // self.stride)

    @property
    def n_toks(self):
        return self.capacity - self.n_refs


class Mlp:
    """Linear -> act -> Linear weights as torch tensors (w1 [hidden, in],
    b1 [hidden] fp32 or None, w2 [out, hidden], b2 [out] fp32 or None)."""

    def __init__(self, w1, b1, w2, b2, act=ACT_GELU):
        self.w1, self.b1, self.w2, self.b2, self.act = w1, b1, w2, b2, act

    @classmethod
    def from_dict(cls, d, act=ACT_GELU, device=None):
        mv = (lambda t: t.to(device)) if device is not None else (lambda t: t)
        return cls(mv(d["w1"]), mv(d["b1"]) if d.get("b1") is not None else None,
                   mv(d["w2"]), mv(d["b2"]) if d.get("b2") is not None else None, act)

    def c(self) -> CMlp:
        return CMlp(_ptr(self.w1), _ptr(self.b1), _ptr(self.w2), _ptr(self.b2),
                    self.w1.shape[1], self.w1.shape[0], self.w2.shape[0], self.act)


class Cache:
    """The four arrays of one (layer, stream) compressed cache, allocated with
    torch on `device` at the sizes deltakv_cache_bytes reports, and its two
    filled lengths (n_built, n_compressed), which the library checks and
    advances; reset() sets them back to 0 to refill the arrays."""

    n_built = 0
    n_compressed = 0

    def __init__(self, shape: Shape, device="cuda"):
        sz = cache_bytes(shape)
        B, H, R, N = shape.batch, shape.num_kv_heads, shape.n_refs, shape.n_toks
        dt = shape.torch_dtype
        self.refs = torch.empty(B, H, R, shape.head_dim, dtype=dt, device=device)
        self.ref_sqnorm = torch.empty(B, H, R, dtype=torch.float32, device=device)
        N = max(N, 0)
        if shape.latent_format == LATENT_Q4:
            # per unit: N rows of d_c / 2 code bytes, then N (shift, scale) bf16 pairs
            self.latents = torch.empty(B, H, N * (shape.d_c // 2 + 4), dtype=torch.uint8,
                                       device=device)
            self.latent_codes = self.latents[:, :, :N * shape.d_c // 2].unflatten(
                2, (N, shape.d_c // 2))
            self.latent_params = self.latents[:, :, N * shape.d_c // 2:].view(
                torch.bfloat16).unflatten(2, (N, 2))
        else:
            self.latents = torch.empty(B, H, N, shape.d_c, dtype=dt, device=device)
        self.idx = torch.empty(B, H, N, shape.k, dtype=torch.uint16, device=device)
        assert self.refs.numel() * self.refs.element_size() == sz["refs"]
        assert self.latents.numel() * self.latents.element_size() == sz["latents"]
        assert self.idx.numel() * 2 == sz["idx"]

    def c(self) -> CCache:
        return CCache(_ptr(self.refs), _ptr(self.ref_sqnorm),
                      _ptr(self.latents) if self.latents.numel() else None,
                      _ptr(self.idx) if self.idx.numel() else None,
                      self.n_built, self.n_compressed, None, 0)

    def _took(self, cc: CCache):
        """Keep the filled lengths the library left in the struct."""
        self.n_built, self.n_compressed = cc.n_built, cc.n_compressed

    def reset(self):
        self.n_built = self.n_compressed = 0

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.refs, self.ref_sqnorm, self.latents, self.idx))


class PagedCache(Cache):
    """A paged cache (shape.page_refs > 0): pools of n_pages pages for the four
    arrays (refs [n_pages, P, d], ref_sqnorm [n_pages, P], latents [n_pages,
    P (s - 1), d_c], idx [n_pages, P (s - 1), k]) and the block table (int32
    [B, H, max_pages] on the device).  The caller assigns pages: write the
    table (e.g. from a free list) before a call touches the positions an
    entry covers."""

    def __init__(self, shape: Shape, n_pages: int, block_table: torch.Tensor, device="cuda"):
        pb = page_bytes(shape)
        P, npp = shape.page_refs, shape.page_refs * (shape.stride - 1)
        dt = shape.torch_dtype
        self.refs = torch.empty(n_pages, P, shape.head_dim, dtype=dt, device=device)
        self.ref_sqnorm = torch.empty(n_pages, P, dtype=torch.float32, device=device)
        self.latents = torch.empty(n_pages, npp, shape.d_c, dtype=dt, device=device)
        self.idx = torch.empty(n_pages, npp, shape.k, dtype=torch.uint16, device=device)
        assert self.refs[0].numel() * self.refs.element_size() == pb["refs"]
        assert self.latents[0].numel() * self.latents.element_size() == pb["latents"]
        if tuple(block_table.shape) != (shape.batch, shape.num_kv_heads, pb["max_pages"]) or \
                block_table.dtype != torch.int32:
            raise ValueError(f"block_table must be int32 [B, H, {pb['max_pages']}]")
        self.block_table = block_table
        self.n_pages = n_pages

    def c(self) -> CCache:
        return CCache(_ptr(self.refs), _ptr(self.ref_sqnorm), _ptr(self.latents),
                      _ptr(self.idx), self.n_built, self.n_compressed, _ptr(self.block_table),
                      self.n_pages)


# --------------------------------------------------------------------- entry points

def cache_bytes(shape: Shape) -> dict:
    vals = [_SZ() for _ in range(4)]
    cs = shape.c()
    _check(lib().deltakv_cache_bytes(ctypes.byref(cs), *[ctypes.byref(v) for v in vals]))
    return dict(zip(("refs", "ref_sqnorm", "latents", "idx"), (v.value for v in vals)))


def page_bytes(shape: Shape) -> dict:
    """Bytes of one page of each pool of a paged shape, and max_pages (the
    block table's row length)."""
    vals = [_SZ() for _ in range(4)]
    mp = ctypes.c_int32()
    cs = shape.c()
    _check(lib().deltakv_page_bytes(ctypes.byref(cs), *[ctypes.byref(v) for v in vals],
                                    ctypes.byref(mp)))
    out = dict(zip(("refs", "ref_sqnorm", "latents", "idx"), (v.value for v in vals)))
    out["max_pages"] = mp.value
    return out


def compress_workspace_bytes(shape: Shape, t0: int, t1: int) -> int:
    v = _SZ()
    cs = shape.c()
    _check(lib().deltakv_compress_workspace_bytes(ctypes.byref(cs), t0, t1, ctypes.byref(v)))
    return v.value


def decode_workspace_bytes(shape: Shape, num_q_heads: int, n_tokens: int) -> int:
    v = _SZ()
    cs = shape.c()
    _check(lib().deltakv_decode_workspace_bytes(ctypes.byref(cs), num_q_heads, n_tokens,
                                                ctypes.byref(v)))
    return v.value


def build_refs(shape: Shape, x: torch.Tensor, t0: int, t1: int, cache: Cache):
    cs, cc = shape.c(), cache.c()
    _check(lib().deltakv_build_refs(ctypes.byref(cs), _ptr(x), t0, t1, ctypes.byref(cc),
                                    _stream()))
    cache._took(cc)


def compress(shape: Shape, x: torch.Tensor, t0: int, t1: int, compressor: Mlp, cache: Cache,
             workspace: Optional[torch.Tensor], stats: Optional[torch.Tensor] = None):
    cs, cm, cc = shape.c(), compressor.c(), cache.c()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().deltakv_compress(ctypes.byref(cs), _ptr(x), t0, t1, ctypes.byref(cm),
                                  ctypes.byref(cc), _ptr(workspace), wsb, _ptr(stats),
                                  _stream()))
    cache._took(cc)


def append_workspace_bytes(shape: Shape, t: int, n_items: int) -> int:
    v = _SZ()
    cs = shape.c()
    _check(lib().deltakv_append_workspace_bytes(ctypes.byref(cs), t, n_items, ctypes.byref(v)))
    return v.value


class AppendBatch:
    """The argument arrays of deltakv_append over a fixed list of caches and
    their compressors, built once; each call passes the position, the new
    rows (one [B, H, 1, d] tensor per cache) and the workspace."""

    def __init__(self, shape: Shape, caches, compressors):
        if len(caches) != len(compressors):
            raise ValueError("one compressor per cache")
        n = len(caches)
        self.shape, self._cs = shape, shape.c()
        self.caches = list(caches)
        self._cc = (CCache * n)(*[c.c() for c in caches])
        self._cm = (CMlp * n)(*[m.c() for m in compressors])
        self._items = (CAppendItem * n)()
        cc0, cm0 = ctypes.addressof(self._cc), ctypes.addressof(self._cm)
        for i in range(n):
            self._items[i].cache = ctypes.cast(cc0 + i * ctypes.sizeof(CCache),
                                               ctypes.POINTER(CCache))
            self._items[i].compressor = ctypes.cast(cm0 + i * ctypes.sizeof(CMlp),
                                                    ctypes.POINTER(CMlp))

    def __call__(self, t: int, xs, workspace: Optional[torch.Tensor]):
        n = len(self.caches)
        if len(xs) != n:
            raise ValueError(f"{len(xs)} rows for {n} caches")
        for i, (x, c) in enumerate(zip(xs, self.caches)):
            self._items[i].x = _ptr(x)
            self._cc[i].n_built, self._cc[i].n_compressed = c.n_built, c.n_compressed
        wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().deltakv_append(ctypes.byref(self._cs), t, n, self._items, _ptr(workspace),
                                    wsb, _stream()))
        for i, c in enumerate(self.caches):
            c._took(self._cc[i])


def append(shape: Shape, t: int, xs, caches, compressors, workspace: Optional[torch.Tensor]):
    """Position t appended to every cache (deltakv_append): xs[i] [B, H, 1, d]
    is the new row of caches[i], compressed with compressors[i]."""
    AppendBatch(shape, caches, compressors)(t, xs, workspace)


def residuals(shape: Shape, x: torch.Tensor, t0: int, t1: int, cache: Cache,
              out: Optional[torch.Tensor]):
    """Residual rows x_p - KV_R(p) of the non-reference positions of [t0, t1)
    into out (fp32 [B, H, n_out, d]; None when there are none)."""
    cs, cc = shape.c(), cache.c()
    _check(lib().deltakv_residuals(ctypes.byref(cs), _ptr(x), t0, t1, ctypes.byref(cc),
                                   _ptr(out), _stream()))


class MlpF32:
    """fp32 master weights of a Linear -> act -> Linear block (w1 [hidden, in],
    b1 [hidden], w2 [out, hidden], b2 [out]), trained in place."""

    def __init__(self, w1, b1, w2, b2, act=ACT_GELU):
        self.w1, self.b1, self.w2, self.b2, self.act = w1, b1, w2, b2, act

    def c(self) -> CMlpF32:
        return CMlpF32(_ptr(self.w1), _ptr(self.b1), _ptr(self.w2), _ptr(self.b2),
                       self.w1.shape[1], self.w1.shape[0], self.w2.shape[0], self.act)


def train_workspace_bytes(compressor: MlpF32, decompressor: MlpF32, n_rows: int):
    """(workspace bytes, packed parameter count) of deltakv_train_step."""
    v, npar = _SZ(), ctypes.c_int64()
    cc, dd = compressor.c(), decompressor.c()
    _check(lib().deltakv_train_workspace_bytes(ctypes.byref(cc), ctypes.byref(dd), n_rows,
                                               ctypes.byref(v), ctypes.byref(npar)))
    return v.value, npar.value


def train_step(delta: torch.Tensor, compressor: MlpF32, decompressor: MlpF32, lr: float,
               workspace: torch.Tensor, momentum: float = 0.0,
               velocity: Optional[torch.Tensor] = None, loss: Optional[torch.Tensor] = None,
               grad: Optional[torch.Tensor] = None, bf16_weights=None):
    """One MSE training step (deltakv_train_step) on delta [n, d] fp32.
    bf16_weights: None or four tensors (or None) receiving bf16 copies of
    W1c, W2c, W1d, W2d."""
    cc, dd = compressor.c(), decompressor.c()
    bw = None
    if bf16_weights is not None:
        bw = (_P * 4)(*[_ptr(t) for t in bf16_weights])
    _check(lib().deltakv_train_step(delta.shape[0], _ptr(delta), ctypes.byref(cc),
                                    ctypes.byref(dd), float(lr), float(momentum),
                                    _ptr(velocity), _ptr(loss), _ptr(grad), bw,
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream()))


def decode_attn(shape: Shape, num_q_heads: int, n_tokens: int, q: torch.Tensor, k_cache: Cache,
                k_dec: Mlp, v_cache: Cache, v_dec: Mlp, scale: float, out: torch.Tensor,
                workspace: Optional[torch.Tensor]):
    cs, kc, km, vc, vm = shape.c(), k_cache.c(), k_dec.c(), v_cache.c(), v_dec.c()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().deltakv_decode_attn(ctypes.byref(cs), num_q_heads, n_tokens, _ptr(q),
                                     ctypes.byref(kc), ctypes.byref(km), ctypes.byref(vc),
                                     ctypes.byref(vm), float(scale), _ptr(out),
                                     _ptr(workspace), wsb, _stream()))


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_attn_noalloc(shape: Shape, num_q_heads: int, n_tokens: int, q: torch.Tensor,
                        k_cache: Cache, k_dec: Mlp, v_cache: Cache, v_dec: Mlp, scale: float,
                        out: torch.Tensor):
    """decode_attn with the library's own per-device scratch (no workspace)."""
    cs, kc, km, vc, vm = shape.c(), k_cache.c(), k_dec.c(), v_cache.c(), v_dec.c()
    _check(lib().deltakv_decode_attn_noalloc(ctypes.byref(cs), num_q_heads, n_tokens, _ptr(q),
                                             ctypes.byref(kc), ctypes.byref(km),
                                             ctypes.byref(vc), ctypes.byref(vm), float(scale),
                                             _ptr(out), _stream()))


def decode_sparse_workspace_bytes(shape: Shape, num_q_heads: int, n_tokens: int,
                                  n_sel: int) -> int:
    v = _SZ()
    cs = shape.c()
    _check(lib().deltakv_decode_sparse_workspace_bytes(ctypes.byref(cs), num_q_heads, n_tokens,
                                                       n_sel, ctypes.byref(v)))
    return v.value


def decode_attn_sparse(shape: Shape, num_q_heads: int, n_tokens: int, q: torch.Tensor,
                       k_cache: Cache, k_dec: Mlp, v_cache: Cache, v_dec: Mlp,
                       positions: torch.Tensor, scale: float, out: torch.Tensor,
                       workspace: Optional[torch.Tensor]):
    """positions: int32 [B, H, n_sel] on the device (n_sel = its last size)."""
    cs, kc, km, vc, vm = shape.c(), k_cache.c(), k_dec.c(), v_cache.c(), v_dec.c()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if positions is not None and positions.dtype != torch.int32:
        raise ValueError("positions must be int32")
    n_sel = int(positions.shape[-1]) if positions is not None else 0
    _check(lib().deltakv_decode_attn_sparse(ctypes.byref(cs), num_q_heads, n_tokens, _ptr(q),
                                            ctypes.byref(kc), ctypes.byref(km), ctypes.byref(vc),
                                            ctypes.byref(vm), _ptr(positions), n_sel,
                                            float(scale), _ptr(out), _ptr(workspace), wsb,
                                            _stream()))


def decode_select_workspace_bytes(shape: Shape, num_q_heads: int, n_tokens: int) -> int:
    v = _SZ()
    cs = shape.c()
    _check(lib().deltakv_decode_select_workspace_bytes(ctypes.byref(cs), num_q_heads, n_tokens,
                                                       ctypes.byref(v)))
    return v.value


def decode_attn_select(shape: Shape, num_q_heads: int, n_tokens: int, q: torch.Tensor,
                       k_cache: Cache, k_dec: Mlp, v_cache: Cache, v_dec: Mlp, scale: float,
                       out: torch.Tensor, positions: torch.Tensor,
                       scores: Optional[torch.Tensor], workspace: Optional[torch.Tensor]):
    """positions: int32 [B, H, n_keep] on the device, written (n_keep = its
    last size); scores: None or fp32 [B, H, n_tokens], written."""
    cs, kc, km, vc, vm = shape.c(), k_cache.c(), k_dec.c(), v_cache.c(), v_dec.c()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if positions is not None and positions.dtype != torch.int32:
        raise ValueError("positions must be int32")
    n_keep = int(positions.shape[-1]) if positions is not None else 0
    _check(lib().deltakv_decode_attn_select(ctypes.byref(cs), num_q_heads, n_tokens, _ptr(q),
                                            ctypes.byref(kc), ctypes.byref(km), ctypes.byref(vc),
                                            ctypes.byref(vm), float(scale), _ptr(out), n_keep,
                                            _ptr(positions), _ptr(scores), _ptr(workspace), wsb,
                                            _stream()))


def decode_window_workspace_bytes(shape: Shape, num_q_heads: int, n_tokens: int,
                                  n_win: int) -> int:
    v = _SZ()
    cs = shape.c()
    _check(lib().deltakv_decode_window_workspace_bytes(ctypes.byref(cs), num_q_heads, n_tokens,
                                                       n_win, ctypes.byref(v)))
    return v.value


def decode_attn_window(shape: Shape, num_q_heads: int, n_tokens: int, q: torch.Tensor,
                       k_cache: Cache, k_dec: Mlp, v_cache: Cache, v_dec: Mlp,
                       k_win: torch.Tensor, v_win: torch.Tensor, scale: float,
                       out: torch.Tensor, workspace: Optional[torch.Tensor]):
    """k_win, v_win: [B, H, n_win, d] exact rows in the shape's dtype."""
    cs, kc, km, vc, vm = shape.c(), k_cache.c(), k_dec.c(), v_cache.c(), v_dec.c()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    n_win = int(k_win.shape[-2]) if k_win is not None else 0
    _check(lib().deltakv_decode_attn_window(ctypes.byref(cs), num_q_heads, n_tokens, _ptr(q),
                                            ctypes.byref(kc), ctypes.byref(km), ctypes.byref(vc),
                                            ctypes.byref(vm), _ptr(k_win), _ptr(v_win), n_win,
                                            float(scale), _ptr(out), _ptr(workspace), wsb,
                                            _stream()))


def decode_varlen_workspace_bytes(shape: Shape, num_q_heads: int, max_tokens: int) -> int:
    v = _SZ()
    cs = shape.c()
    _check(lib().deltakv_decode_varlen_workspace_bytes(ctypes.byref(cs), num_q_heads, max_tokens,
                                                       ctypes.byref(v)))
    return v.value


def decode_attn_varlen(shape: Shape, num_q_heads: int, lengths: torch.Tensor,
                       max_tokens: int, q: torch.Tensor, k_cache: Cache, k_dec: Mlp,
                       v_cache: Cache, v_dec: Mlp, scale: float, out: torch.Tensor,
                       workspace: Optional[torch.Tensor]):
    """lengths: int64 [B] on the device, the tokens each sequence holds (read
    by the kernels); max_tokens: an upper bound of every length."""
    cs, kc, km, vc, vm = shape.c(), k_cache.c(), k_dec.c(), v_cache.c(), v_dec.c()
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if lengths is not None and lengths.dtype != torch.int64:
        raise ValueError("lengths must be int64")
    _check(lib().deltakv_decode_attn_varlen(ctypes.byref(cs), num_q_heads, _ptr(lengths),
                                            int(max_tokens), _ptr(q),
                                            ctypes.byref(kc), ctypes.byref(km), ctypes.byref(vc),
                                            ctypes.byref(vm), float(scale), _ptr(out),
                                            _ptr(workspace), wsb, _stream()))


PEAK_MFMA_BF16, PEAK_GELU_F16 = 0, 1


def peak_probe(kind: int, blocks: int, iters: int, sink: torch.Tensor):
    """Measurement helper: enqueue the matrix-core or GELU rate loop."""
    _check(lib().deltakv_peak_probe(kind, blocks, iters, _ptr(sink), _stream()))


def status_string(status: int) -> str:
    return lib().deltakv_status_string(status).decode()


def last_error() -> str:
    return lib().deltakv_last_error().decode()


def version() -> str:
    return lib().deltakv_version().decode()


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A 256-byte aligned device buffer of at least nbytes (torch allocation)."""
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


deltakv_cache_bytes = cache_bytes
deltakv_compress_workspace_bytes = compress_workspace_bytes
deltakv_decode_workspace_bytes = decode_workspace_bytes
deltakv_build_refs = build_refs
deltakv_compress = compress
deltakv_decode_attn = decode_attn
deltakv_decode_attn_noalloc = decode_attn_noalloc
deltakv_decode_sparse_workspace_bytes = decode_sparse_workspace_bytes
deltakv_decode_attn_sparse = decode_attn_sparse
deltakv_decode_select_workspace_bytes = decode_select_workspace_bytes
deltakv_decode_attn_select = decode_attn_select
deltakv_decode_window_workspace_bytes = decode_window_workspace_bytes
deltakv_decode_attn_window = decode_attn_window
deltakv_decode_varlen_workspace_bytes = decode_varlen_workspace_bytes
deltakv_decode_attn_varlen = decode_attn_varlen
deltakv_peak_probe = peak_probe
deltakv_status_string = status_string
deltakv_last_error = last_error
deltakv_version = version
