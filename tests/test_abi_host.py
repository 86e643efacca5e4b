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


def _cache(addr=0x10000, filled=4096):
    """A cache stand-in whose first `filled` positions count as built and
    compressed (the decode calls read at most that many)."""
    c = dk.Cache.__new__(dk.Cache)
    c.refs = c.ref_sqnorm = c.latents = c.idx = _FakePtr(addr)
    c.n_built = c.n_compressed = filled
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
        dk.compress(sh, x, 0, 16, _mlp(128, 256, 16), _cache(filled=0), None)  # wrong d_c
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        dk.compress(sh, x, 0, 16, _mlp(128, 100, 32), _cache(filled=0), None)  # hidden 100
    assert e.value.status == 2


def _fresh(n_built=0, n_compressed=0):
    c = _cache(filled=0)
    c.n_built, c.n_compressed = n_built, n_compressed
    return c


def test_build_refs_is_append_only():
    # references are built in order: t0 must be the filled length, which the
    # library advances only on success
    sh = _shape(capacity=4096)
    x = _FakePtr()
    for c, t0 in ((_fresh(), 16), (_fresh(64, 64), 0), (_fresh(64, 64), 128)):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.build_refs(sh, x, t0, t0 + 16, c)
        assert e.value.status == 1 and "n_built" in e.value.detail
        assert c.n_built in (0, 64)
    with pytest.raises(dk.DeltaKVError) as e:     # inconsistent filled lengths
        dk.build_refs(sh, x, 64, 80, _fresh(64, 65))
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        dk.build_refs(sh, x, 4097, 4098, _fresh(4097, 0))
    assert e.value.status in (1, 3)


def test_compress_needs_built_references_and_the_next_range():
    sh = _shape(capacity=4096)
    x = _FakePtr()
    ws = _FakePtr(0x30000, 1 << 30)
    comp = _mlp(128, 256, 32)
    # positions whose references were never built
    c = _fresh(n_built=1024, n_compressed=0)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.compress(sh, x, 0, 2048, comp, c, ws)
    assert e.value.status == 1 and "n_built" in e.value.detail
    assert c.n_compressed == 0
    # a range that does not start at the compressed length (a gap, or a redo)
    for t0 in (512, 0):
        c = _fresh(n_built=2048, n_compressed=256)
        with pytest.raises(dk.DeltaKVError) as e:
            dk.compress(sh, x, t0, 1024, comp, c, ws)
        assert e.value.status == 1 and "n_compressed" in e.value.detail
        assert c.n_compressed == 256
    # a range of references only: nothing to compute, the length still advances
    c = _fresh(n_built=33, n_compressed=32)
    dk.compress(sh, x, 32, 33, comp, c, ws)
    assert c.n_compressed == 33


def test_decode_reads_only_compressed_positions():
    sh = _shape(capacity=4096)
    dec = _mlp(32, 256, 128)
    ws = _FakePtr(0x30000, 1 << 30)
    for kf, vf in ((4095, 4096), (4096, 1000)):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.decode_attn(sh, 32, 4096, _FakePtr(), _cache(filled=kf), dec, _cache(filled=vf),
                           dec, 0.088, _FakePtr(), ws)
        assert e.value.status == 1 and "compressed" in e.value.detail


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


class _FakeLens(_FakePtr):
    """An int64 [B] device length array stand-in."""

    def __init__(self, addr=0x80000):
        super().__init__(addr, 8 * 3)
        import torch
        self.dtype = torch.int64


def test_varlen_length_errors_return_before_any_launch():
    sh = _shape(capacity=4096, batch=3)
    dec = _mlp(32, 256, 128)
    need = dk.decode_varlen_workspace_bytes(sh, 32, 4096)

    def call(lens, max_tokens, ws=_FakePtr(0x30000, need), filled=4096):
        dk.decode_attn_varlen(sh, 32, lens, max_tokens, _FakePtr(), _cache(filled=filled), dec,
                              _cache(filled=filled), dec, 0.088, _FakePtr(), ws)

    for max_tokens, status in ((0, 1), (4097, 3)):
        with pytest.raises(dk.DeltaKVError) as e:
            call(_FakeLens(), max_tokens)
        assert e.value.status == status
    with pytest.raises(dk.DeltaKVError) as e:
        call(None, 4096)
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakeLens(0x80004), 4096)                  # misaligned lengths
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakeLens(), 4096, filled=4000)            # past the compressed length
    assert e.value.status == 1
    with pytest.raises(dk.DeltaKVError) as e:
        call(_FakeLens(), 4096, ws=_FakePtr(0x30000, need - 1))
    assert e.value.status == 4


def test_noalloc_decode_rejects_calls_beyond_its_scratch():
    # batch 64 x 8 KV heads at 128k needs more than the 64 MiB the
    # allocation-free entry point holds; the call fails before touching a device
    sh = _shape(batch=64, capacity=131072)
    assert dk.decode_workspace_bytes(sh, 32, 131072) > dk.NOALLOC_SCRATCH_BYTES
    assert dk.decode_workspace_bytes(_shape(capacity=131072), 32, 131072) < \
        dk.NOALLOC_SCRATCH_BYTES
    dec = _mlp(32, 256, 128)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.decode_attn_noalloc(sh, 32, 131072, _FakePtr(), _cache(filled=131072), dec,
                               _cache(filled=131072), dec, 0.088, _FakePtr())
    assert e.value.status == 4 and "scratch" in e.value.detail


def _append_items(n, t, base=0x100000):
    caches = []
    for i in range(n):
        c = _cache(addr=base + i * 0x1000, filled=0)
        c.n_built = c.n_compressed = t
        caches.append(c)
    return caches, [_mlp(128, 256, 32) for _ in range(n)]


def test_append_checks_every_item_before_anything_is_enqueued():
    sh = _shape(capacity=4096)
    ws = _FakePtr(0x30000, 1 << 30)
    t = 1001                                   # not a reference position (s = 16)
    # one cache behind the others: the call fails and no length moves
    caches, comps = _append_items(5, t)
    caches[3].n_compressed = t - 1
    with pytest.raises(dk.DeltaKVError) as e:
        dk.append(sh, t, [_FakePtr()] * 5, caches, comps, ws)
    assert e.value.status == 1 and "items[3]" in e.value.detail
    assert [c.n_built for c in caches] == [t] * 5
    assert [c.n_compressed for c in caches] == [t, t, t, t - 1, t]
    # the same cache twice
    caches, comps = _append_items(3, t)
    caches[2] = caches[0]
    with pytest.raises(dk.DeltaKVError) as e:
        dk.append(sh, t, [_FakePtr()] * 3, caches, comps, ws)
    assert e.value.status == 1 and "same cache" in e.value.detail
    # a misaligned row, a wrong compressor, a too-small workspace
    caches, comps = _append_items(2, t)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.append(sh, t, [_FakePtr(), _FakePtr(0x10008)], caches, comps, ws)
    assert e.value.status == 1 and "items[1].x" in e.value.detail
    comps[1] = _mlp(128, 256, 16)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.append(sh, t, [_FakePtr()] * 2, caches, comps, ws)
    assert e.value.status == 1
    caches, comps = _append_items(2, t)
    need = dk.append_workspace_bytes(sh, t, 2)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.append(sh, t, [_FakePtr()] * 2, caches, comps, _FakePtr(0x30000, need - 1))
    assert e.value.status == 4
    assert all(c.n_built == t and c.n_compressed == t for c in caches)


def test_append_position_and_item_count_limits():
    sh = _shape(capacity=4096)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.append_workspace_bytes(sh, 4096, 4)       # position past the capacity
    assert e.value.status == 3
    for n in (0, 4097):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.append_workspace_bytes(sh, 100, n)
        assert e.value.status == 1
    caches, comps = _append_items(2, 50)
    with pytest.raises(dk.DeltaKVError) as e:          # caches at 50, position 51
        dk.append(sh, 51, [_FakePtr()] * 2, caches, comps, _FakePtr(0x30000, 1 << 30))
    assert e.value.status == 1 and "n_built == n_compressed" in e.value.detail


@pytest.mark.parametrize("kw", [dict(capacity=131072 + 1024, stride=8, k=8, d_c=16),
                                dict(capacity=9000, stride=5, k=3, head_dim=64, num_kv_heads=2),
                                dict(capacity=5000, stride=16, batch=3, dtype=dk.F32),
                                dict(capacity=40000, stride=16, page_refs=128)])
def test_append_workspace_covers_the_per_cache_compress_and_never_shrinks(kw):
    # a workspace sized for the last position serves every earlier one,
    # reference positions included
    sh = _shape(**kw)
    cap = sh.capacity
    ts = sorted(set(list(range(0, min(cap, 700))) + list(range(0, cap, 97)) +
                    list(range(cap - 40, cap))))
    for n in (1, 7, 64):
        prev = 0
        for t in ts:
            w = dk.append_workspace_bytes(sh, t, n)
            assert w >= prev, (n, t)
            if t % sh.stride:
                assert w >= dk.compress_workspace_bytes(sh, t, t + 1)
            prev = w


# ---- paged layout -------------------------------------------------------------------


def test_paged_page_sizes_and_shape_checks():
    sh = _shape(page_refs=256)                 # stride 16: 4096 positions per page
    pb = dk.page_bytes(sh)
    assert pb["refs"] == 256 * 128 * 2 and pb["ref_sqnorm"] == 256 * 4
    assert pb["latents"] == 256 * 15 * 32 * 2 and pb["idx"] == 256 * 15 * 4 * 2
    assert pb["max_pages"] == 32768 // 4096
    full = dk.cache_bytes(sh)                  # every logical page of every unit backed
    for a in ("refs", "ref_sqnorm", "latents", "idx"):
        assert full[a] == 8 * pb["max_pages"] * pb[a]
    # a ragged capacity: the last page is partly used
    assert dk.page_bytes(_shape(page_refs=128, capacity=5000))["max_pages"] == 3
    with pytest.raises(dk.DeltaKVError) as e:  # not a paged shape
        dk.page_bytes(_shape())
    assert e.value.status == 1
    for bad in (dict(page_refs=100), dict(page_refs=64), dict(page_refs=8192),
                dict(page_refs=256, stride=1), dict(page_refs=256, dtype=dk.F32),
                dict(page_refs=256, latent_format=dk.LATENT_Q4)):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.page_bytes(_shape(**bad))
        assert e.value.status == 2, bad


def _pcache(addr=0x10000, filled=4096, table=0x50000, n_pages=64):
    c = dk.PagedCache.__new__(dk.PagedCache)
    c.refs = c.ref_sqnorm = c.latents = c.idx = _FakePtr(addr)
    c.block_table = _FakePtr(table) if table else None
    c.n_pages = n_pages
    c.n_built = c.n_compressed = filled
    return c


def test_paged_cache_arguments_checked_before_any_launch():
    sh = _shape(capacity=4096, page_refs=128)
    x = _FakePtr()
    for c in (_pcache(filled=0, table=0), _pcache(filled=0, table=0x50002),
              _pcache(filled=0, n_pages=0)):
        with pytest.raises(dk.DeltaKVError) as e:
            dk.build_refs(sh, x, 0, 16, c)
        assert e.value.status == 1 and ("block_table" in e.value.detail or
                                        "n_pages" in e.value.detail)
    dec = _mlp(32, 256, 128)
    ws = _FakePtr(0x30000, 1 << 30)
    # K and V must share one block table
    with pytest.raises(dk.DeltaKVError) as e:
        dk.decode_attn(sh, 32, 4096, _FakePtr(), _pcache(), dec, _pcache(table=0x60000), dec,
                       0.088, _FakePtr(), ws)
    assert e.value.status == 2 and "block table" in e.value.detail
    # shapes the wave-specialised decode does not cover
    sh3 = _shape(capacity=4096, page_refs=128, k=3)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.decode_attn(sh3, 32, 4096, _FakePtr(), _pcache(), dec, _pcache(), dec, 0.088,
                       _FakePtr(), ws)
    assert e.value.status == 2
    # calls without a paged path
    with pytest.raises(dk.DeltaKVError) as e:
        dk.decode_attn_sparse(sh, 32, 4096, _FakePtr(), _pcache(), dec, _pcache(), dec,
                              _FakePos(64), 0.088, _FakePtr(), ws)
    assert e.value.status == 2
    with pytest.raises(dk.DeltaKVError) as e:
        dk.residuals(sh, x, 0, 64, _pcache(), _FakePtr())
    assert e.value.status == 2
    # a reference pool beyond 2 GiB (65536 pages of 128 rows of 256 bytes)
    with pytest.raises(dk.DeltaKVError) as e:
        dk.build_refs(sh, x, 0, 16, _pcache(filled=0, n_pages=65537))
    assert e.value.status == 2 and "2 GiB" in e.value.detail


def test_paged_compress_workspace_holds_the_staged_rows():
    # a paged compress stages the unit's references and the range's index
    # and latent rows ahead of the unit-contiguous call's own workspace
    for t0, t1 in ((0, 131072), (65536, 69632), (100000, 100001)):
        pg = dk.compress_workspace_bytes(_shape(capacity=131072, page_refs=256), t0, t1)
        ct = dk.compress_workspace_bytes(_shape(capacity=131072), t0, t1)
        R = -(-t1 // 16)
        nq = (t1 - R) - (t0 - -(-t0 // 16))
        staged = 8 * (R * 128 * 2 + R * 4 + nq * 4 * 2 + nq * 32 * 2)
        assert pg >= ct + staged, (t0, t1)
        assert pg <= ct + staged + 4 * 256 * 8 + 4 * 256, (t0, t1)
