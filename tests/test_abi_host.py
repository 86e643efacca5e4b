"""Host-side checks of libdeltakv.so (no GPU needed): the library loads, exports
every entry point declared in include/deltakv.h, sizes its arrays by the
closed forms, and rejects bad arguments before touching the device."""
import ctypes
import json
import os
import re

import pytest

import decode_attention_deltakv_amd as dk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "deltakv.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(deltakv_[a-z_]+)\(",
                                 text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert len(names) >= 9, names
    lib = ctypes.CDLL(dk.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in deltakv.h but not exported"


def test_version_and_status_strings():
    assert "gfx950" in dk.version()
    assert dk.status_string(0) == "DELTAKV_OK"
    assert dk.status_string(4) == "DELTAKV_ERR_WORKSPACE"


def _shape(**kw):
    base = dict(batch=1, num_kv_heads=8, head_dim=128, stride=16, k=4, d_c=32, capacity=32768,
                dtype=dk.BF16)
    base.update(kw)
    return dk.Shape(**base)


def test_cache_bytes_closed_form():
    sh = _shape()
    sz = dk.cache_bytes(sh)
    R, N = 2048, 30720
    assert sz["refs"] == 8 * R * 128 * 2
    assert sz["ref_sqnorm"] == 8 * R * 4
    assert sz["latents"] == 8 * N * 32 * 2
    assert sz["idx"] == 8 * N * 4 * 2
    # ragged capacity, fp32, stride 3
    sh = _shape(capacity=100, stride=3, dtype=dk.F32, head_dim=64, d_c=16, k=2,
                num_kv_heads=1)
    sz = dk.cache_bytes(sh)
    assert sz["refs"] == 34 * 64 * 4 and sz["latents"] == 66 * 16 * 4 and sz["idx"] == 66 * 2 * 2


def test_uncompressed_size_from_the_pages_and_compressed_ratio():
    # DeltaKV summary, section 1: Llama-3.1-8B at 128k context and batch 8
    # needs more than 130 GB of KV cache
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "llama31_8b_kv_size.json")))
    full = g["batch"] * g["T"] * g["layers"] * g["kv_heads"] * g["head_dim"] * 2 * 2
    assert full == g["expected_bytes"] > g["page_lower_bound_bytes"]
    sh = _shape(batch=8, capacity=131072)
    sz = dk.cache_bytes(sh)
    per_layer_stream = sz["refs"] + sz["latents"] + sz["idx"]
    compressed = per_layer_stream * 2 * g["layers"]
    assert compressed == 8 * 8 * 2 * 32 * 10944512  # units x (refs + latents + idx)
    assert 0.32 < compressed / full < 0.33


def test_stride_one_has_no_compressed_tokens():
    sz = dk.cache_bytes(_shape(stride=1, capacity=1000))
    assert sz["latents"] == 0 and sz["idx"] == 0


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=96), 2), (dict(head_dim=0), 2), (dict(k=0), 2), (dict(k=9), 2),
    (dict(d_c=24), 2), (dict(stride=0), 1), (dict(capacity=0), 1), (dict(batch=0), 1),
    (dict(dtype=7), 2), (dict(stride=2, capacity=2 * 65535 + 1), 3),
])
def test_bad_shapes_rejected(bad, status):
    with pytest.raises(dk.DeltaKVError) as e:
        dk.cache_bytes(_shape(**bad))
    assert e.value.status == status
    assert dk.last_error()


def test_largest_capacity_accepted():
    sz = dk.cache_bytes(_shape(stride=2, capacity=2 * 65535, num_kv_heads=1))
    assert sz["refs"] == 65535 * 128 * 2


class _FakePtr:
    """A tensor stand-in: only data_ptr / numel are used by the binding."""

    def __init__(self, addr=0x10000, n=16):
        self.addr, self.n = addr, n

    def data_ptr(self):
        return self.addr

    def is_contiguous(self):
        return True

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def _cache(addr=0x10000):
    c = dk.Cache.__new__(dk.Cache)
    c.refs = c.ref_sqnorm = c.latents = c.idx = _FakePtr(addr)
    return c


def _mlp(din, h, dout, addr=0x20000):
    m = dk.Mlp(_FakePtr(addr), None, _FakePtr(addr), None)
    m.c = lambda: dk.CMlp(addr, None, addr, None, din, h, dout, 0)
    return m


def test_range_and_pointer_errors_return_before_any_launch():
    sh = _shape(capacity=4096)
    x = _FakePtr()
    with pytest.raises(dk.DeltaKVError) as e:
        dk.build_refs(sh, x, 10, 10, _cache())
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        dk.build_refs(sh, x, 0, 4097, _cache())
    assert e.value.status == 3
    with pytest.raises(dk.DeltaKVError) as e:
        dk.build_refs(sh, _FakePtr(0x10008), 0, 16, _cache())   # misaligned x
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        dk.compress(sh, x, 0, 16, _mlp(128, 256, 16), _cache(), None)  # wrong d_c
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        dk.compress(sh, x, 0, 16, _mlp(128, 100, 32), _cache(), None)  # hidden 100
    assert e.value.status == 2


def test_workspace_too_small_is_reported():
    sh = _shape(capacity=4096)
    need = dk.decode_workspace_bytes(sh, 32, 4096)
    assert need > 0
    ws = _FakePtr(0x30000, need - 1)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.decode_attn(sh, 32, 4096, _FakePtr(), _cache(), _mlp(32, 256, 128), _cache(),
                       _mlp(32, 256, 128), 0.088, _FakePtr(), ws)
    assert e.value.status == 4


def test_decode_head_grouping_checked():
    sh = _shape(capacity=4096)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.decode_workspace_bytes(sh, 12, 4096)     # not a multiple of 8
    assert e.value.status == 2
    with pytest.raises(dk.DeltaKVError) as e:
        dk.decode_workspace_bytes(sh, 72, 4096)     # 9 query heads per KV head
    assert e.value.status == 2
    with pytest.raises(dk.DeltaKVError):
        dk.decode_workspace_bytes(sh, 32, 0)


class _FakePos(_FakePtr):
    """An int32 [B, H, n_sel] position-list stand-in."""

    def __init__(self, n_sel, addr=0x40000):
        super().__init__(addr, 4 * n_sel)
        import torch
        self.dtype = torch.int32
        self.shape = (1, 8, n_sel)


def test_sparse_workspace_grows_with_the_list_and_adds_to_the_dense_tables():
    sh = _shape(capacity=131072)
    small = dk.decode_sparse_workspace_bytes(sh, 32, 131072, 1024)
    big = dk.decode_sparse_workspace_bytes(sh, 32, 131072, 8192)
    assert 0 < small < big
    # the split lists alone: two int32 lists of n_sel per unit
    assert big - small >= 2 * 8 * (8192 - 1024) * 4
    for bad in (0, -3, (1 << 20) + 1):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.decode_sparse_workspace_bytes(sh, 32, 131072, bad)
        assert e.value.status == 1


def test_sparse_decode_argument_errors_return_before_any_launch():
    sh = _shape(capacity=4096)
    dec = _mlp(32, 256, 128)
    need = dk.decode_sparse_workspace_bytes(sh, 32, 4096, 64)
    ok_ws = _FakePtr(0x30000, need)

    def call(pos, ws=ok_ws, n_tokens=4096, hq=32):
        dk.decode_attn_sparse(sh, hq, n_tokens, _FakePtr(), _cache(), dec, _cache(), dec, pos,
                              0.088, _FakePtr(), ws)

    with pytest.raises(dk.DeltaKVError) as e:
        call(None)                                   # no list
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakePos(64, addr=0x40004))             # misaligned list
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakePos(64), ws=_FakePtr(0x30000, need - 1))
    assert e.value.status == 4
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakePos(64), n_tokens=4097)
    assert e.value.status == 3
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakePos(64), hq=36)
    assert e.value.status == 2
    with pytest.raises(ValueError):
        p = _FakePos(64)
        import torch
        p.dtype = torch.int64
        call(p)


def test_select_argument_errors_return_before_any_launch():
    sh = _shape(capacity=4096)
    dec = _mlp(32, 256, 128)
    need = dk.decode_select_workspace_bytes(sh, 32, 4096)
    assert need > dk.decode_workspace_bytes(sh, 32, 4096)
    ok_ws = _FakePtr(0x30000, need)

    def call(pos, ws=ok_ws, scores=None):
        dk.decode_attn_select(sh, 32, 4096, _FakePtr(), _cache(), dec, _cache(), dec, 0.088,
                              _FakePtr(), pos, scores, ws)

    with pytest.raises(dk.DeltaKVError) as e:
        call(None)                                       # no output list
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakePos(64), scores=_FakePtr(0x50004))     # misaligned scores
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakePos(64), ws=_FakePtr(0x30000, need - 1))
    assert e.value.status == 4
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakePos((1 << 20) + 1))                    # n_keep too large
    assert e.value.status == 1


def test_q4_latent_bytes_and_unsupported_combinations():
    sh = _shape(latent_format=dk.LATENT_Q4)
    sz = dk.cache_bytes(sh)
    assert sz["latents"] == 8 * 30720 * (32 // 2 + 4)          # codes + (shift, scale)
    assert sz["refs"] == dk.cache_bytes(_shape())["refs"]
    with pytest.raises(dk.DeltaKVError) as e:
        dk.cache_bytes(_shape(latent_format=2))
    assert e.value.status == 1
    for bad in (dict(dtype=dk.F32), dict(d_c=64)):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.cache_bytes(_shape(latent_format=dk.LATENT_Q4, **bad))
        assert e.value.status == 2
    x = _FakePtr()
    with pytest.raises(dk.DeltaKVError) as e:  # no 4-bit writer for hidden 64
        dk.compress(_shape(latent_format=dk.LATENT_Q4, capacity=4096), x, 0, 16,
                    _mlp(128, 64, 32), _cache(), _FakePtr(0x30000, 1 << 20))
    assert e.value.status == 2
    sh3 = _shape(latent_format=dk.LATENT_Q4, capacity=4096, k=3)
    dec = _mlp(32, 256, 128)
    with pytest.raises(dk.DeltaKVError) as e:  # no 4-bit reader for k = 3
        dk.decode_attn(sh3, 32, 4096, _FakePtr(), _cache(), dec, _cache(), dec, 0.088,
                       _FakePtr(), _FakePtr(0x30000, 1 << 30))
    assert e.value.status == 2


def test_window_argument_errors_return_before_any_launch():
    sh = _shape(capacity=4096)
    dec = _mlp(32, 256, 128)
    need = dk.decode_window_workspace_bytes(sh, 32, 4096, 100)
    assert need > dk.decode_workspace_bytes(sh, 32, 4096)
    for bad in (0, 65536):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.decode_window_workspace_bytes(sh, 32, 4096, bad)
        assert e.value.status == 1

    class _Win(_FakePtr):
        shape = (1, 8, 100, 128)

    def call(kw, vw, ws=_FakePtr(0x30000, need)):
        dk.decode_attn_window(sh, 32, 4096, _FakePtr(), _cache(), dec, _cache(), dec, kw, vw,
                              0.088, _FakePtr(), ws)

    with pytest.raises(dk.DeltaKVError) as e:
        call(_Win(0x60000), None)
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_Win(0x60008), _Win(0x70000))               # misaligned window rows
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_Win(0x60000), _Win(0x70000), ws=_FakePtr(0x30000, need - 1))
    assert e.value.status == 4


def test_varlen_length_errors_return_before_any_launch():
    sh = _shape(capacity=4096, batch=3)
    dec = _mlp(32, 256, 128)
    need = dk.decode_varlen_workspace_bytes(sh, 32, 4096)
    for bad, status in (((10, 0, 5), 1), ((10, 4097, 5), 3)):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.decode_attn_varlen(sh, 32, bad, _FakePtr(), _cache(), dec, _cache(), dec, 0.088,
                                  _FakePtr(), _FakePtr(0x30000, need))
        assert e.value.status == status
    with pytest.raises(dk.DeltaKVError) as e:
        dk.decode_attn_varlen(sh, 32, (10, 4096, 5), _FakePtr(), _cache(), dec, _cache(), dec,
                              0.088, _FakePtr(), _FakePtr(0x30000, need - 1))
    assert e.value.status == 4
