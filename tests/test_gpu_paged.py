"""GPU parity of the paged cache layout (DeltaKV page, section 4: a cache
manager for irregular compressed layouts; the block-table layout of paged KV
caches for batched serving).

A paged cache is built and compressed through a random block table (pages of
every unit scattered over a pool shared by all units): row for row, read back
through the table, it must hold bit for bit what the unit-contiguous cache
holds after the same calls (reference rows, squared norms, index lists,
latents), and every decode call over it (dense, allocation-free, mixed
lengths, with a window, with token selection) must return bit for bit the
contiguous call's result.  The contiguous path is checked against the oracle
elsewhere; one paged decode per case is also compared with the oracle here,
on the rows read back through the table (bf16 bar TOL)."""
import math

import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
import oracle
from deltakv_synth import queries
from parity import (TOL, gpu_mlp, idx_to_oracle, make_kv, make_mlp, oracle_mlp, rel_err_rows,
                    say, to_np)

pytestmark = pytest.mark.gpu


def _table(shape, seed, spare=3):
    """A block table naming distinct pool pages in random order, and the pool
    size (a few pages more than the table uses)."""
    mp = dk.page_bytes(shape)["max_pages"]
    U = shape.batch * shape.num_kv_heads
    n_pages = U * mp + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)[:U * mp].to(torch.int32)
    return perm.reshape(shape.batch, shape.num_kv_heads, mp).cuda(), n_pages


def _logical(pc, shape, n_refs, n_toks):
    """The arrays of a paged cache read back through its table, unit by unit,
    in the unit-contiguous shapes [B, H, rows, ...]."""
    P = shape.page_refs
    npp = P * (shape.stride - 1)
    tbl = pc.block_table.cpu().long()
    B, H = shape.batch, shape.num_kv_heads
    j = torch.arange(n_refs)
    q = torch.arange(n_toks)
    refs, sqn, lat, idx = [], [], [], []
    rp, sp, lp, ip = pc.refs.cpu(), pc.ref_sqnorm.cpu(), pc.latents.cpu(), pc.idx.cpu()
    for b in range(B):
        for h in range(H):
            pr = tbl[b, h][j // P]
            pt = tbl[b, h][q // npp]
            refs.append(rp[pr, j % P])
            sqn.append(sp[pr, j % P])
            lat.append(lp[pt, q % npp])
            idx.append(ip[pt, q % npp])
    st = lambda xs: torch.stack(xs).reshape(B, H, *xs[0].shape)
    return st(refs), st(sqn), st(lat), st(idx)


def _same_bits(a, b, what):
    a, b = a.cpu(), b.cpu()
    if a.dtype in (torch.bfloat16, torch.uint16):
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    bad = (a != b)
    assert not bad.any(), f"{what}: {int(bad.sum())} entries differ"


def _grow(shape, xg, caches, comp, bounds, appends):
    """Chunked build + compress over `bounds`, then one-token appends of the
    positions in `appends` (deltakv_append over every cache at once)."""
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        ws = dk.workspace(dk.compress_workspace_bytes(shape, t0, t1))
        for x, c in zip(xg, caches):
            xc = x[:, :, t0:t1].contiguous()
            dk.build_refs(shape, xc, t0, t1, c)
            dk.compress(shape, xc, t0, t1, comp, c, ws)
    batch = dk.AppendBatch(shape, caches, [comp] * len(caches))
    for t in appends:
        ws = dk.workspace(dk.append_workspace_bytes(shape, t, len(caches)))
        batch(t, [x[:, :, t:t + 1].contiguous() for x in xg], ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [
    # (B, H, G, d, s, k, dc, hid, page_refs, bounds, n_appends)
    (2, 2, 4, 128, 16, 4, 32, 256, 128, (0, 1500, 4100, 4990), 10),
    (1, 3, 8, 64, 8, 8, 16, 128, 256, (0, 6000), 5),
], ids=["llama-k4-chunks", "k8-d64-one-call"])
def test_paged_cache_matches_contiguous_bitwise(cfg):
    B, H, G, d, s, k, dc, hid, P, bounds, n_app = cfg
    T = bounds[-1] + n_app
    seed = 900 + T
    say(f"[case] paged {cfg}")
    cshape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    pshape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16, 0, P)
    kx = make_kv(B, H, T, d, torch.bfloat16, key=(seed, 0))
    vx = make_kv(B, H, T, d, torch.bfloat16, key=(seed, 1))
    xg = [kx.cuda(), vx.cuda()]
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(seed, 10), bias_std=0.05)
    comp = gpu_mlp(cw, dk.ACT_GELU)
    cc = [dk.Cache(cshape), dk.Cache(cshape)]
    tbl, n_pages = _table(pshape, seed)
    pc = [dk.PagedCache(pshape, n_pages, tbl), dk.PagedCache(pshape, n_pages, tbl)]
    for c in pc:  # pages start as garbage: every row read must have been written
        for t in (c.refs, c.latents):
            t.view(torch.int16).fill_(-1)
        c.ref_sqnorm.fill_(float("nan"))
        c.idx.view(torch.int16).fill_(-1)
    apps = list(range(bounds[-1], T))
    _grow(cshape, xg, cc, comp, list(bounds), apps)
    _grow(pshape, xg, pc, comp, list(bounds), apps)
    R, N = oracle.num_refs(T, s), T - oracle.num_refs(T, s)
    for name, c, p in zip(("K", "V"), cc, pc):
        refs, sqn, lat, idx = _logical(p, pshape, R, N)
        _same_bits(refs, c.refs[:, :, :R], f"{name} reference rows")
        _same_bits(sqn, c.ref_sqnorm[:, :, :R], f"{name} squared norms")
        _same_bits(idx, c.idx[:, :, :N], f"{name} index lists")
        _same_bits(lat, c.latents[:, :, :N], f"{name} latents")

    kd = gpu_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(seed, 12), bias_std=0.05)[0],
                 dk.ACT_GELU)
    vd = gpu_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(seed, 13), bias_std=0.05)[0],
                 dk.ACT_GELU)
    Hq, scale = H * G, 1.0 / math.sqrt(d)
    q = queries(B * Hq, d, key=(seed, 20), dtype=torch.bfloat16).reshape(B, Hq, d).cuda()

    def run(shape, kc, vc, call):
        out = torch.full((B, Hq, d), float("nan"), device="cuda")
        extra = call(shape, kc, vc, out)
        torch.cuda.synchronize()
        return out, extra

    def dense(shape, kc, vc, out):
        dk.decode_attn(shape, Hq, T, q, kc, kd, vc, vd, scale, out,
                       dk.workspace(dk.decode_workspace_bytes(shape, Hq, T)))

    def noalloc(shape, kc, vc, out):
        dk.decode_attn_noalloc(shape, Hq, T - 7, q, kc, kd, vc, vd, scale, out)

    lens = torch.tensor([T - 3 * i * 311 for i in range(B)], dtype=torch.int64, device="cuda")

    def varlen(shape, kc, vc, out):
        dk.decode_attn_varlen(shape, Hq, lens, T, q, kc, kd, vc, vd, scale, out,
                              dk.workspace(dk.decode_varlen_workspace_bytes(shape, Hq, T)))

    kw = make_kv(B, H, 37, d, torch.bfloat16, key=(seed, 30)).cuda()
    vw = make_kv(B, H, 37, d, torch.bfloat16, key=(seed, 31)).cuda()

    def window(shape, kc, vc, out):
        dk.decode_attn_window(shape, Hq, T, q, kc, kd, vc, vd, kw, vw, scale, out,
                              dk.workspace(dk.decode_window_workspace_bytes(shape, Hq, T, 37)))

    def select(shape, kc, vc, out):
        pos = torch.empty(B, H, 300, dtype=torch.int32, device="cuda")
        sc = torch.empty(B, H, T, dtype=torch.float32, device="cuda")
        dk.decode_attn_select(shape, Hq, T, q, kc, kd, vc, vd, scale, out, pos, sc,
                              dk.workspace(dk.decode_select_workspace_bytes(shape, Hq, T)))
        return pos, sc

    for name, call in (("dense", dense), ("noalloc", noalloc), ("varlen", varlen),
                       ("window", window), ("select", select)):
        oc, ec = run(cshape, cc[0], cc[1], call)
        op, ep = run(pshape, pc[0], pc[1], call)
        _same_bits(op, oc, f"{name} decode output")
        if ec is not None:
            for a, b in zip(ep, ec):
                _same_bits(a, b, f"{name} selection")
        say(f"[case] paged {cfg}: {name} bitwise equal")

    # the paged dense decode against the oracle on the rows read back through
    # the table, for one KV head
    out, _ = run(pshape, pc[0], pc[1], dense)
    kl, vl = _logical(pc[0], pshape, R, N), _logical(pc[1], pshape, R, N)
    b, h = B - 1, H - 1
    want = oracle.decode_head(to_np(q[b, h * G:(h + 1) * G].cpu()), to_np(kl[0][b, h]),
                              to_np(kl[2][b, h]), idx_to_oracle(kl[3][b, h]),
                              oracle_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(seed, 12),
                                                  bias_std=0.05)[0], dk.ACT_GELU),
                              to_np(vl[0][b, h]), to_np(vl[2][b, h]), idx_to_oracle(vl[3][b, h]),
                              oracle_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(seed, 13),
                                                  bias_std=0.05)[0], dk.ACT_GELU),
                              T, s, scale)
    err = rel_err_rows(out[b, h * G:(h + 1) * G].cpu().double().numpy(), want)
    say(f"[case] paged {cfg}: decode vs oracle rel err {err:.3e}")
    assert err <= TOL[dk.BF16]


def test_paged_units_of_different_lengths_share_one_pool():
    # two sequences of very different lengths take pages from one pool as
    # they grow (pages handed out in order of need, interleaved between the
    # sequences); the short one's table row names pages only for what it
    # holds, the rest of its row points at page 0 of another unit (never
    # read: the mixed-length decode stops at each length)
    B, H, G, d, s, k, dc, hid, P = 2, 2, 4, 128, 16, 4, 32, 256, 128
    lens = (5100, 1300)
    T = max(lens)
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16, 0, P)
    cshape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    mp = dk.page_bytes(shape)["max_pages"]
    ppos = P * s
    need = [[-(-L // ppos)] * H for L in lens]
    tbl = torch.zeros(B, H, mp, dtype=torch.int32)
    nxt = 0
    for i in range(mp):
        for b in range(B):
            for h in range(H):
                if i < need[b][h]:
                    tbl[b, h, i] = nxt
                    nxt += 1
    n_pages = nxt
    say(f"[case] paged mixed lengths {lens}: {n_pages} pages for {B * H * mp} logical")
    seed = 950
    kx = make_kv(B, H, T, d, torch.bfloat16, key=(seed, 0)).cuda()
    vx = make_kv(B, H, T, d, torch.bfloat16, key=(seed, 1)).cuda()
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(seed, 10), bias_std=0.05)
    comp = gpu_mlp(cw, dk.ACT_GELU)
    tg = tbl.cuda()
    pk, pv = dk.PagedCache(shape, n_pages, tg), dk.PagedCache(shape, n_pages, tg)
    ck, cv = dk.Cache(cshape), dk.Cache(cshape)
    for c in (ck, cv):  # rows past a sequence's length: defined, never attended
        for t in (c.refs, c.ref_sqnorm, c.latents, c.idx):
            t.view(torch.uint8).zero_()
    # each sequence is compressed to its own length by a batch-1 call whose
    # block table is that sequence's row (its pages in the shared pools); the
    # contiguous cache gets the same rows from batch-1 contiguous calls
    for b, L in enumerate(lens):
        sb = dk.Shape(1, H, d, s, k, dc, T, dk.BF16, 0, P)
        sbc = dk.Shape(1, H, d, s, k, dc, T, dk.BF16)
        tb = tg[b:b + 1].contiguous()
        for x, c_all, pc_all in ((kx, ck, pk), (vx, cv, pv)):
            xb = x[b:b + 1, :, :L].contiguous()
            one = dk.PagedCache(sb, n_pages, tb)
            one.refs, one.ref_sqnorm, one.latents, one.idx = (pc_all.refs, pc_all.ref_sqnorm,
                                                              pc_all.latents, pc_all.idx)
            onec = dk.Cache(sbc)
            for cc_, sh in ((one, sb), (onec, sbc)):
                dk.build_refs(sh, xb, 0, L, cc_)
                dk.compress(sh, xb, 0, L, comp, cc_, dk.workspace(
                    dk.compress_workspace_bytes(sh, 0, L)))
            torch.cuda.synchronize()
            R, N = oracle.num_refs(L, s), L - oracle.num_refs(L, s)
            c_all.refs[b, :, :R] = onec.refs[0, :, :R]
            c_all.ref_sqnorm[b, :, :R] = onec.ref_sqnorm[0, :, :R]
            c_all.latents[b, :, :N] = onec.latents[0, :, :N]
            c_all.idx[b, :, :N] = onec.idx[0, :, :N]
    for c in (pk, pv, ck, cv):
        c.n_built = c.n_compressed = T
    kd = gpu_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(seed, 12))[0], dk.ACT_GELU)
    vd = gpu_mlp(make_mlp(dc, hid, d, torch.bfloat16, key=(seed, 13))[0], dk.ACT_GELU)
    Hq, scale = H * G, 1.0 / math.sqrt(d)
    q = queries(B * Hq, d, key=(seed, 20), dtype=torch.bfloat16).reshape(B, Hq, d).cuda()
    L = torch.tensor(lens, dtype=torch.int64, device="cuda")
    outs = []
    for sh, a, v in ((shape, pk, pv), (cshape, ck, cv)):
        out = torch.full((B, Hq, d), float("nan"), device="cuda")
        dk.decode_attn_varlen(sh, Hq, L, T, q, a, kd, v, vd, scale, out,
                              dk.workspace(dk.decode_varlen_workspace_bytes(sh, Hq, T)))
        torch.cuda.synchronize()
        outs.append(out)
    _same_bits(outs[0], outs[1], "mixed-length paged decode")
    assert torch.isfinite(outs[0]).all()


def test_paged_llama_layer_128k_equals_contiguous():
    # one layer of the Llama-3.1-8B-shaped 128k workload at full size, in the
    # launch configuration the benchmark times (one compress call per stream,
    # one decode call), into paged caches (pages of 128 references = 2048
    # positions, shuffled over the pool) and into contiguous ones: the stored
    # rows read back through the table and the decode output equal bit for bit
    # (the contiguous layer is checked against the oracle in test_gpu_parity)
    from deltakv_synth import WORKLOADS, kv_rows, unit_key, workload_index, xavier_mlp
    w = WORKLOADS["llama8b-32layer-T128k-bf16"]
    widx = workload_index(w.name)
    B, H, G, T, d, s = 1, w.kv_heads, w.q_heads // w.kv_heads, w.T, w.head_dim, w.stride
    cshape = dk.Shape(B, H, d, s, w.k, w.d_c, T, dk.BF16)
    pshape = dk.Shape(B, H, d, s, w.k, w.d_c, T, dk.BF16, 0, 128)
    tbl, n_pages = _table(pshape, 77)
    say(f"[case] paged llama8b-T128k one layer: {n_pages} pages per cache")
    cc, pc = [], []
    for st in (0, 1):
        x = torch.stack([kv_rows(T, d, w.n_dirs, w.n_centroids, key=unit_key(widx, 0, 0, h, st),
                                 dtype=torch.bfloat16, device="cuda") for h in range(H)])[None]
        comp = gpu_mlp(xavier_mlp(d, w.hidden, w.d_c, key=(1, widx, 0, st),
                                  dtype=torch.bfloat16), dk.ACT_GELU)
        for sh, cache, out in ((cshape, dk.Cache(cshape), cc),
                               (pshape, dk.PagedCache(pshape, n_pages, tbl), pc)):
            dk.build_refs(sh, x, 0, T, cache)
            dk.compress(sh, x, 0, T, comp, cache,
                        dk.workspace(dk.compress_workspace_bytes(sh, 0, T)))
            out.append(cache)
        torch.cuda.synchronize()
        del x
    R, N = oracle.num_refs(T, s), T - oracle.num_refs(T, s)
    for name, c, p in zip(("K", "V"), cc, pc):
        refs, sqn, lat, idx = _logical(p, pshape, R, N)
        _same_bits(refs, c.refs, f"{name} reference rows")
        _same_bits(sqn, c.ref_sqnorm, f"{name} squared norms")
        _same_bits(idx, c.idx, f"{name} index lists")
        _same_bits(lat, c.latents, f"{name} latents")
    kd = gpu_mlp(xavier_mlp(w.d_c, w.hidden, d, key=(2, widx, 0, 0), dtype=torch.bfloat16),
                 dk.ACT_GELU)
    vd = gpu_mlp(xavier_mlp(w.d_c, w.hidden, d, key=(2, widx, 0, 1), dtype=torch.bfloat16),
                 dk.ACT_GELU)
    q = queries(H * G, d, key=(3, widx), dtype=torch.bfloat16).reshape(B, H * G, d).cuda()
    outs = []
    for sh, caches in ((cshape, cc), (pshape, pc)):
        out = torch.full((B, H * G, d), float("nan"), device="cuda")
        dk.decode_attn(sh, H * G, T, q, caches[0], kd, caches[1], vd, 1.0 / math.sqrt(d), out,
                       dk.workspace(dk.decode_workspace_bytes(sh, H * G, T)))
        torch.cuda.synchronize()
        outs.append(out)
    _same_bits(outs[1], outs[0], "128k paged decode output")
    say("[case] paged llama8b-T128k: arrays and decode output bitwise equal")
