"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Indices must match bit for bit (rank order and unused
slots included); latents and attention outputs must be within the stated
tolerance (max over rows of max|g - o| / max|o|: 2e-2 for bf16, 1e-4 for
fp32).  Decode is checked on the GPU's own stored cache, so each stage is
compared on identical inputs."""
import math

import numpy as np
import pytest
import torch

import decode_attention_deltakv_amd as dk
import oracle
from deltakv_synth import WORKLOADS, kv_rows, queries, xavier_mlp
from parity import (TOL, check_compress_unit, gpu_compress, gpu_decode, gpu_mlp, make_kv,
                    make_mlp, oracle_decode_head, oracle_mlp, rel_err_rows, say, to_np)

pytestmark = pytest.mark.gpu


def _run_case(name, B, H, G, T, d, s, k, dc, hid, dtype, seed, bias_std=0.0, chunks=None,
              n_dirs=8, n_centroids=64, positions=None, decode_heads=None):
    say(f"[case] {name}: B={B} H={H} G={G} T={T} d={d} s={s} k={k} dc={dc} hid={hid} "
        f"dtype={dtype} seed={seed}")
    tdt = torch.float32 if dtype == dk.F32 else torch.bfloat16
    shape = dk.Shape(B, H, d, s, k, dc, T, dtype)
    kx = make_kv(B, H, T, d, tdt, key=(seed, 0), n_dirs=n_dirs, n_centroids=n_centroids)
    vx = make_kv(B, H, T, d, tdt, key=(seed, 1), n_dirs=n_dirs, n_centroids=n_centroids)
    kcw, _ = make_mlp(d, hid, dc, tdt, key=(seed, 10), bias_std=bias_std)
    vcw, _ = make_mlp(d, hid, dc, tdt, key=(seed, 11), bias_std=bias_std)
    kdw, _ = make_mlp(dc, hid, d, tdt, key=(seed, 12), bias_std=bias_std)
    vdw, _ = make_mlp(dc, hid, d, tdt, key=(seed, 13), bias_std=bias_std)
    kc = gpu_compress(shape, kx, gpu_mlp(kcw, dk.ACT_GELU), chunks)
    vc = gpu_compress(shape, vx, gpu_mlp(vcw, dk.ACT_GELU), chunks)
    tol = TOL[dtype]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            worst = max(worst, check_compress_unit(shape, kx[b, h], kc, b, h,
                                                   oracle_mlp(kcw, dk.ACT_GELU), positions, tol))
            worst = max(worst, check_compress_unit(shape, vx[b, h], vc, b, h,
                                                   oracle_mlp(vcw, dk.ACT_GELU), positions, tol))
    Hq = H * G
    q = queries(B * Hq, d, key=(seed, 20), dtype=tdt).reshape(B, Hq, d)
    scale = 1.0 / math.sqrt(d)
    out = gpu_decode(shape, Hq, T, q, kc, gpu_mlp(kdw, dk.ACT_GELU), vc,
                     gpu_mlp(vdw, dk.ACT_GELU), scale)
    derr = 0.0
    heads = [(b, h) for b in range(B) for h in range(H)] if decode_heads is None else decode_heads
    for b, h in heads:
        want = oracle_decode_head(shape, T, to_np(q[b, h * G:(h + 1) * G]), kc, vc, b, h,
                                  oracle_mlp(kdw, dk.ACT_GELU), oracle_mlp(vdw, dk.ACT_GELU),
                                  scale)
        derr = max(derr, rel_err_rows(out[b, h * G:(h + 1) * G], want))
    say(f"[case] {name}: latent rel err {worst:.3e}, decode rel err {derr:.3e}")
    assert derr <= tol, f"decode rel err {derr} > {tol}"
    return kc, vc, out


def test_tiny_single_head_fp32():
    w = WORKLOADS["tiny-1head-T512-fp32"]
    _run_case("tiny-1head-T512-fp32", 1, 1, 1, w.T, w.head_dim, w.stride, w.k, w.d_c, w.hidden,
              dk.F32, seed=1, n_dirs=w.n_dirs, n_centroids=w.n_centroids)


def test_bf16_llama_heads_ragged():
    # several token tiles, ragged tail, two sequences, GQA 4
    _run_case("bf16-llama-heads-ragged", 2, 2, 4, 1000, 128, 16, 4, 32, 256, dk.BF16, seed=2,
              bias_std=0.05)


@pytest.mark.parametrize("cfg", [
    # (d, s, k, dc, hid, G, T, dtype)
    (128, 8, 8, 16, 256, 4, 777, dk.BF16),    # streaming workload's shapes
    (128, 8, 6, 32, 256, 4, 1200, dk.BF16),   # k > 4 with d_c = 32 in the Compressor
    (64, 8, 8, 32, 128, 8, 1300, dk.BF16),    # k = 8 wave-specialised decode, 8 heads per KV head
    (64, 3, 2, 64, 64, 1, 500, dk.BF16),
    (64, 5, 5, 128, 128, 8, 301, dk.BF16),
    (64, 4, 3, 64, 128, 2, 999, dk.BF16),     # matrix-core decode at head_dim 64
    (128, 16, 4, 32, 128, 4, 1500, dk.BF16),
    (128, 16, 4, 32, 256, 2, 600, dk.F32),
    (64, 2, 1, 16, 128, 4, 257, dk.F32),
    # k = 4 and d_c <= 32: the wave-specialised decode kernel
    (64, 16, 4, 16, 256, 8, 1100, dk.BF16),
    (128, 8, 4, 32, 256, 1, 900, dk.BF16),
    (128, 16, 4, 16, 128, 3, 2000, dk.BF16),
    (64, 4, 4, 32, 128, 2, 45, dk.BF16),       # a single partial tile
])
def test_shape_variants(cfg):
    d, s, k, dc, hid, G, T, dtype = cfg
    _run_case(f"variant-{cfg}", 1, 2, G, T, d, s, k, dc, hid, dtype, seed=3 + s + k)


@pytest.mark.parametrize("cfg", [
    # (B, H, G, T, d, s, k, dc, hid, dtype)
    (3, 2, 4, 1100, 128, 16, 4, 32, 256, dk.BF16),   # wave-specialised decode
    (2, 3, 2, 700, 64, 8, 8, 16, 128, dk.BF16),      # four-wave decode, k = 8
    (2, 2, 4, 300, 64, 16, 4, 16, 128, dk.F32),      # general (fp32) paths
    (8, 8, 4, 1536, 128, 16, 4, 32, 256, dk.BF16),   # batch 8, all KV heads
])
def test_batched_sequences(cfg):
    # several sequences in one call: every (sequence, KV head) unit of the
    # compression and every query head of the decode against the oracle
    B, H, G, T, d, s, k, dc, hid, dtype = cfg
    _run_case(f"batch-{cfg}", B, H, G, T, d, s, k, dc, hid, dtype, seed=130 + B + d,
              bias_std=0.05)


def test_streaming_chunks_match_offline_bitwise():
    B, H, T, d, s, k, dc, hid = 1, 2, 700, 128, 8, 8, 16, 256
    say(f"[case] streaming: T={T}")
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    x = make_kv(B, H, T, d, torch.bfloat16, key=(40, 0))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(40, 1))
    comp = gpu_mlp(cw, dk.ACT_GELU)
    off = gpu_compress(shape, x, comp)
    bounds = [0, 100, 357, 358, 359, 360, 512, 513, 600] + list(range(601, 700, 9)) + [700]
    ch = gpu_compress(shape, x, comp, chunks=sorted(set(bounds)))
    for name in ("refs", "ref_sqnorm", "latents", "idx"):
        a, b = getattr(off, name), getattr(ch, name)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name


def test_short_prefixes_and_single_token_context():
    # tokens with fewer than k candidates (sentinel slots), and decode over
    # T = 1 (only reference 0) and T = 2
    B, H, G, d, s, k, dc, hid = 1, 1, 4, 64, 16, 4, 16, 128
    _run_case("short-prefix", B, H, G, 40, d, s, k, dc, hid, dk.BF16, seed=50)
    for T in (1, 2, 17):
        _run_case(f"tiny-context-{T}", B, H, G, T, d, s, k, dc, hid, dk.F32, seed=51 + T)


def test_stride_one_is_dense_attention():
    B, H, G, T, d = 1, 2, 4, 300, 128
    say("[case] stride-1")
    shape = dk.Shape(B, H, d, 1, 4, 32, T, dk.BF16)
    kx = make_kv(B, H, T, d, torch.bfloat16, key=(60, 0))
    vx = make_kv(B, H, T, d, torch.bfloat16, key=(60, 1))
    cw, _ = make_mlp(d, 256, 32, torch.bfloat16, key=(60, 2))
    dw, _ = make_mlp(32, 256, d, torch.bfloat16, key=(60, 3))
    kc = gpu_compress(shape, kx, gpu_mlp(cw, 0))
    vc = gpu_compress(shape, vx, gpu_mlp(cw, 0))
    q = queries(B * H * G, d, key=(60, 4), dtype=torch.bfloat16).reshape(B, H * G, d)
    out = gpu_decode(shape, H * G, T, q, kc, gpu_mlp(dw, 0), vc, gpu_mlp(dw, 0), 1 / math.sqrt(d))
    for h in range(H):
        want = oracle.attention(to_np(q[0, h * G:(h + 1) * G]), to_np(kx[0, h]), to_np(vx[0, h]),
                                1 / math.sqrt(d))
        assert rel_err_rows(out[0, h * G:(h + 1) * G], want) <= 2e-2


@pytest.mark.parametrize("dtype", [dk.F32, dk.BF16])
def test_orthogonal_identity_pair_gives_dense_attention(dtype):
    # identity activation, d_c = hidden = head_dim, W1c = Q, W2c = I,
    # W1d = Q^T, W2d = I: the rebuilt cache is the input, so decode equals
    # dense attention on the original K / V
    B, H, G, T, d, s, k = 1, 2, 4, 640, 64, 16, 4
    say(f"[case] orthogonal pair dtype={dtype}")
    tdt = torch.float32 if dtype == dk.F32 else torch.bfloat16
    shape = dk.Shape(B, H, d, s, k, d, T, dtype)
    kx = make_kv(B, H, T, d, tdt, key=(70, 0))
    vx = make_kv(B, H, T, d, tdt, key=(70, 1))
    Q, _ = np.linalg.qr(np.random.default_rng(70).standard_normal((d, d)))
    Qt = torch.from_numpy(Q).to(tdt)
    eye = torch.eye(d).to(tdt)
    comp = dk.Mlp(Qt.contiguous().cuda(), None, eye.cuda(), None, dk.ACT_IDENTITY)
    dec = dk.Mlp(Qt.T.contiguous().cuda(), None, eye.cuda(), None, dk.ACT_IDENTITY)
    kc = gpu_compress(shape, kx, comp)
    vc = gpu_compress(shape, vx, comp)
    q = queries(B * H * G, d, key=(70, 2), dtype=tdt).reshape(B, H * G, d)
    out = gpu_decode(shape, H * G, T, q, kc, dec, vc, dec, 1 / math.sqrt(d))
    for h in range(H):
        want = oracle.attention(to_np(q[0, h * G:(h + 1) * G]), to_np(kx[0, h]), to_np(vx[0, h]),
                                1 / math.sqrt(d))
        err = rel_err_rows(out[0, h * G:(h + 1) * G], want)
        say(f"  head {h}: rel err vs dense attention {err:.3e}")
        assert err <= TOL[dtype]


def test_duplicate_reference_rows_break_ties_by_position():
    B, H, T, d, s, k = 1, 1, 400, 128, 8, 4
    say("[case] duplicate refs")
    x = make_kv(B, H, T, d, torch.bfloat16, key=(80, 0))
    # make references 3, 10, 20, 33 identical, and several tokens equal to them
    for j in (10, 20, 33):
        x[0, 0, j * s] = x[0, 0, 3 * s]
    for p in (3 * s + 1, 21 * s + 5, 40 * s + 7, 49 * s + 3):
        x[0, 0, p] = x[0, 0, 3 * s]
    shape = dk.Shape(B, H, d, s, k, 32, T, dk.BF16)
    cw, _ = make_mlp(d, 256, 32, torch.bfloat16, key=(80, 1))
    c = gpu_compress(shape, x, gpu_mlp(cw, 0))
    check_compress_unit(shape, x[0, 0], c, 0, 0, oracle_mlp(cw, 0), tol=2e-2)
    q = lambda p: (p // s) * (s - 1) + (p % s) - 1
    assert c.idx[0, 0, q(40 * s + 7)].tolist() == [3, 10, 20, 33]
    assert c.idx[0, 0, q(21 * s + 5)].tolist()[:3] == [3, 10, 20]


def test_repeat_runs_are_bitwise_identical():
    B, H, G, T, d, s, k, dc, hid = 1, 2, 4, 900, 128, 16, 4, 32, 256
    say("[case] determinism")
    kc1, vc1, out1 = _run_case("determinism-a", B, H, G, T, d, s, k, dc, hid, dk.BF16, seed=90)
    kc2, vc2, out2 = _run_case("determinism-b", B, H, G, T, d, s, k, dc, hid, dk.BF16, seed=90)
    for a, b in ((kc1, kc2), (vc1, vc2)):
        for name in ("refs", "latents", "idx"):
            assert torch.equal(getattr(a, name).view(torch.uint8), getattr(b, name).view(torch.uint8))
    assert np.array_equal(out1, out2)


def test_llama_layer_32k_sampled():
    # the one-layer Llama-3.1-8B-shaped workload at full size: every unit is
    # compressed on the GPU; the oracle checks sampled tokens per unit (first
    # and last 64 compressed tokens plus 128 random ones) and decode on two
    # KV heads (8 query heads) over all 32768 tokens
    w = WORKLOADS["llama8b-1layer-T32k-bf16"]
    T, s = w.T, w.stride
    nonref = oracle.nonref_positions(T, s)
    rng = np.random.default_rng(7)
    pos = np.unique(np.concatenate([nonref[:64], nonref[-64:],
                                    rng.choice(nonref, 128, replace=False)]))
    _run_case("llama8b-1layer-T32k-bf16 sampled", 1, w.kv_heads, w.q_heads // w.kv_heads, T,
              w.head_dim, s, w.k, w.d_c, w.hidden, dk.BF16, seed=100, n_dirs=w.n_dirs,
              n_centroids=w.n_centroids, positions=pos, decode_heads=[(0, 0), (0, 7)])


def test_long_reference_ranges_checked_everywhere():
    # every token of a 12288-token context with stride 8 (up to 1536
    # candidate references per token, 48 reference blocks of the top-k
    # search), compared index for index with the oracle
    _run_case("long-reference-ranges", 1, 1, 4, 12288, 128, 8, 4, 32, 256, dk.BF16, seed=60,
              n_dirs=8, n_centroids=256)


def test_long_reference_ranges_in_chunks_k8():
    # the prompt compressed in 2048-token chunks with k = 8: later chunks see
    # up to 1536 references in few token tiles, so the top-k search splits
    # each tile's reference range over several blocks and merges their lists
    _run_case("long-reference-ranges-chunks-k8", 1, 1, 4, 12288, 128, 8, 8, 16, 256, dk.BF16,
              seed=61, n_dirs=8, n_centroids=256, chunks=list(range(0, 12288 + 1, 2048)))


def test_exact_ties_beyond_candidate_list_take_exact_fallback():
    # 12 identical reference rows (more than the approximate candidate list
    # keeps) and tokens equal to them: the certificate cannot separate the
    # tied references, so those tokens are rescanned exactly; the result must
    # still be the lowest ordinals, and the fallback counter must see them
    B, H, T, d, s, k = 1, 1, 600, 128, 8, 4
    say("[case] fallback via exact ties")
    x = make_kv(B, H, T, d, torch.bfloat16, key=(110, 0))
    dup = [2, 5, 9, 11, 14, 20, 23, 30, 31, 40, 47, 55]
    for j in dup:
        x[0, 0, j * s] = x[0, 0, 2 * s]
    tie_pos = [56 * s + 3, 60 * s + 1, 70 * s + 6, 74 * s + 2]
    for p in tie_pos:
        x[0, 0, p] = x[0, 0, 2 * s]
    shape = dk.Shape(B, H, d, s, k, 32, T, dk.BF16)
    cw, _ = make_mlp(d, 256, 32, torch.bfloat16, key=(110, 1))
    stats = torch.zeros(4, dtype=torch.int32, device="cuda")
    c = gpu_compress(shape, x, gpu_mlp(cw, 0), stats=stats)
    check_compress_unit(shape, x[0, 0], c, 0, 0, oracle_mlp(cw, 0), tol=2e-2)
    q = lambda p: (p // s) * (s - 1) + (p % s) - 1
    for p in tie_pos:
        assert c.idx[0, 0, q(p)].tolist() == dup[:4]
    n_fb = int(stats[0].item())
    say(f"  fallback tokens: {n_fb}")
    assert n_fb >= len(tie_pos)


def test_near_tied_references_take_split_and_block_fallbacks():
    # every reference row is one base row with one coordinate moved by a
    # single bf16 step: all distances of a token differ by far less than the
    # certificate's error terms, so (nearly) every token goes to the exact
    # fallback scan; 3840 listed tokens exceed the entries whose scan is split
    # over blocks, so the per-token block scan takes the rest.  Every token
    # is compared with the oracle.
    B, H, T, d, s, k = 1, 1, 4096, 128, 16, 4
    say("[case] near-tied references: split and block fallback scans")
    x = make_kv(B, H, T, d, torch.bfloat16, key=(120, 0))
    base = x[0, 0, 0].clone()
    g = torch.Generator().manual_seed(120)
    for j in range(T // s):
        row = base.clone()
        c = int(torch.randint(0, d, (1,), generator=g))
        f = row[c].float()
        step = torch.tensor(float(f) * (1 + 2.0 ** -7) if int(torch.randint(0, 2, (1,), generator=g))
                            else float(f) * (1 - 2.0 ** -7)).to(torch.bfloat16)
        row[c] = step
        x[0, 0, j * s] = row
    shape = dk.Shape(B, H, d, s, k, 32, T, dk.BF16)
    cw, _ = make_mlp(d, 256, 32, torch.bfloat16, key=(120, 1))
    stats = torch.zeros(4, dtype=torch.int32, device="cuda")
    c = gpu_compress(shape, x, gpu_mlp(cw, 0), stats=stats)
    n_fb = int(stats[0].item())
    say(f"  fallback tokens: {n_fb}")
    check_compress_unit(shape, x[0, 0], c, 0, 0, oracle_mlp(cw, 0), tol=2e-2)
    assert n_fb > 1024


def test_decode_graph_replays_match_eager():
    # decode captured in a HIP graph (as a serving loop would), replayed several
    # times with eager library work and synchronisations between the replays;
    # every replay must equal the eager result bit for bit
    B, H, G, T, d, s, k, dc, hid = 1, 2, 4, 1500, 128, 16, 4, 32, 256
    say("[case] decode graph replay")
    tdt = torch.bfloat16
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    kx = make_kv(B, H, T, d, tdt, key=(120, 0))
    vx = make_kv(B, H, T, d, tdt, key=(120, 1))
    kc = gpu_compress(shape, kx, gpu_mlp(make_mlp(d, hid, dc, tdt, key=(120, 2))[0], 0))
    vc = gpu_compress(shape, vx, gpu_mlp(make_mlp(d, hid, dc, tdt, key=(120, 3))[0], 0))
    kd = gpu_mlp(make_mlp(dc, hid, d, tdt, key=(120, 4))[0], 0)
    vd = gpu_mlp(make_mlp(dc, hid, d, tdt, key=(120, 5))[0], 0)
    Hq = H * G
    scale = 1.0 / math.sqrt(d)
    qa = queries(B * Hq, d, key=(120, 6), dtype=tdt).reshape(B, Hq, d).cuda()
    qb = queries(B * Hq, d, key=(120, 7), dtype=tdt).reshape(B, Hq, d).cuda()
    ws = dk.workspace(dk.decode_workspace_bytes(shape, Hq, T))
    ws2 = dk.workspace(dk.decode_workspace_bytes(shape, Hq, T))
    out_e = torch.empty(B, Hq, d, dtype=torch.float32, device="cuda")
    dk.decode_attn(shape, Hq, T, qa, kc, kd, vc, vd, scale, out_e, ws)
    torch.cuda.synchronize()
    out_g = torch.empty_like(out_e)
    out_o = torch.empty_like(out_e)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dk.decode_attn(shape, Hq, T, qa, kc, kd, vc, vd, scale, out_g, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep} differs from eager"
        # eager work on another query between replays
        dk.decode_attn(shape, Hq, T, qb, kc, kd, vc, vd, scale, out_o, ws2)
        torch.cuda.synchronize()
    say("  4 replays equal to eager")


def test_single_token_appends_over_many_references_match_offline():
    # one-token appends at the end of a context with many references (the
    # exact per-token scan with the references split over several blocks)
    # must store the same indices and latents as one offline call
    B, H, T, d, s, k, dc, hid = 1, 2, 1600, 128, 2, 8, 16, 256
    say(f"[case] appends: T={T} s={s} k={k}")
    shape = dk.Shape(B, H, d, s, k, dc, T, dk.BF16)
    x = make_kv(B, H, T, d, torch.bfloat16, key=(130, 0))
    cw, _ = make_mlp(d, hid, dc, torch.bfloat16, key=(130, 1))
    comp = gpu_mlp(cw, dk.ACT_GELU)
    off = gpu_compress(shape, x, comp)
    bounds = [0, T - 41] + list(range(T - 40, T + 1))
    ap = gpu_compress(shape, x, comp, chunks=bounds)
    for name in ("refs", "ref_sqnorm", "latents", "idx"):
        a, b = getattr(off, name), getattr(ap, name)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
    tail = [p for p in range(T - 40, T) if p % s != 0]
    check_compress_unit(shape, x[0, 1], ap, 0, 1, oracle_mlp(cw, dk.ACT_GELU),
                        positions=np.array(tail), tol=2e-2)


def test_llama_layer_128k_sampled():
    # one layer of the benchmark's Llama-3.1-8B-shaped 128k workload, in the
    # launch configuration the benchmark times (one compress call per stream
    # over the whole prefix, one decode call): inputs generated on the GPU,
    # the oracle checks sampled tokens of two units (first / last 64 and 128
    # random compressed positions: index lists bit-exact, latents within
    # 2e-2) and the decode of one KV head over all 131072 positions
    from deltakv_synth import WORKLOADS, workload_index, unit_key
    w = WORKLOADS["llama8b-32layer-T128k-bf16"]
    widx = workload_index(w.name)
    B, H, G, T, d, s = 1, w.kv_heads, w.q_heads // w.kv_heads, w.T, w.head_dim, w.stride
    shape = dk.Shape(B, H, d, s, w.k, w.d_c, T, dk.BF16)
    say("[case] llama8b-T128k one layer: generating and compressing on the GPU")
    xs, caches, comps = [], [], []
    for st in (0, 1):
        x = torch.stack([kv_rows(T, d, w.n_dirs, w.n_centroids, key=unit_key(widx, 0, 0, h, st),
                                 dtype=torch.bfloat16, device="cuda") for h in range(H)])[None]
        cw = xavier_mlp(d, w.hidden, w.d_c, key=(1, widx, 0, st), dtype=torch.bfloat16)
        cache = dk.Cache(shape)
        dk.build_refs(shape, x, 0, T, cache)
        ws = dk.workspace(dk.compress_workspace_bytes(shape, 0, T))
        dk.compress(shape, x, 0, T, gpu_mlp(cw, dk.ACT_GELU), cache, ws)
        torch.cuda.synchronize()
        xs.append(x.cpu())
        caches.append(cache)
        comps.append(cw)
        del x, ws
    nonref = oracle.nonref_positions(T, s)
    rng = np.random.default_rng(11)
    pos = np.unique(np.concatenate([nonref[:64], nonref[-64:],
                                    rng.choice(nonref, 128, replace=False)]))
    worst = 0.0
    for st in (0, 1):
        for h in (0, 7):
            worst = max(worst, check_compress_unit(shape, xs[st][0, h], caches[st], 0, h,
                                                   oracle_mlp(comps[st], dk.ACT_GELU), pos,
                                                   TOL[dk.BF16]))
    say(f"[case] llama8b-T128k: sampled latent rel err {worst:.3e}")
    kdw = xavier_mlp(w.d_c, w.hidden, d, key=(2, widx, 0, 0), dtype=torch.bfloat16)
    vdw = xavier_mlp(w.d_c, w.hidden, d, key=(2, widx, 0, 1), dtype=torch.bfloat16)
    q = queries(H * G, d, key=(3, widx), dtype=torch.bfloat16).reshape(B, H * G, d)
    scale = 1.0 / math.sqrt(d)
    out = gpu_decode(shape, H * G, T, q, caches[0], gpu_mlp(kdw, dk.ACT_GELU), caches[1],
                     gpu_mlp(vdw, dk.ACT_GELU), scale)
    h = 3
    want = oracle_decode_head(shape, T, to_np(q[0, h * G:(h + 1) * G]), caches[0], caches[1], 0,
                              h, oracle_mlp(kdw, dk.ACT_GELU), oracle_mlp(vdw, dk.ACT_GELU), scale)
    err = rel_err_rows(out[0, h * G:(h + 1) * G], want)
    say(f"[case] llama8b-T128k: decode rel err {err:.3e} (KV head {h})")
    assert err <= TOL[dk.BF16]


def test_streaming_llama_layer_128k_sampled():
    # one layer of the streaming workload at full size: a 131072-token prompt
    # compressed in 4096-token chunks (references accumulate across chunks, up
    # to 16384 per unit at stride 8), then 8 one-token appends, as the
    # benchmark launches them; the oracle checks sampled tokens (prompt and
    # every appended token) of two units per stream and the decode of one KV
    # head over all 131080 positions
    from deltakv_synth import WORKLOADS, workload_index, unit_key
    w = WORKLOADS["llama8b-32layer-T128k-stream-s8k8-bf16"]
    widx = workload_index(w.name)
    A = 8
    B, H, G, T, d, s = 1, w.kv_heads, w.q_heads // w.kv_heads, w.T, w.head_dim, w.stride
    cap = T + A
    shape = dk.Shape(B, H, d, s, w.k, w.d_c, cap, dk.BF16)
    say("[case] stream-s8k8 one layer: generating, chunked compression, appends")
    xs, caches, comps = [], [], []
    for st in (0, 1):
        x = torch.stack([kv_rows(cap, d, w.n_dirs, w.n_centroids, key=unit_key(widx, 0, 0, h, st),
                                 dtype=torch.bfloat16, device="cuda") for h in range(H)])[None]
        cw = xavier_mlp(d, w.hidden, w.d_c, key=(1, widx, 0, st), dtype=torch.bfloat16)
        cm = gpu_mlp(cw, dk.ACT_GELU)
        cache = dk.Cache(shape)
        ws = dk.workspace(max(dk.compress_workspace_bytes(shape, a, b_)
                              for a, b_ in [(c0, min(T, c0 + w.chunk)) for c0 in range(0, T, w.chunk)]
                              + [(cap - 1, cap)]))
        bounds = list(range(0, T, w.chunk)) + [T] + list(range(T + 1, cap + 1))
        for t0, t1 in zip(bounds[:-1], bounds[1:]):
            xc = x[:, :, t0:t1].contiguous()
            dk.build_refs(shape, xc, t0, t1, cache)
            dk.compress(shape, xc, t0, t1, cm, cache, ws)
        torch.cuda.synchronize()
        xs.append(x.cpu())
        caches.append(cache)
        comps.append(cw)
        del x, ws
    nonref = oracle.nonref_positions(cap, s)
    rng = np.random.default_rng(12)
    pos = np.unique(np.concatenate([nonref[:64], nonref[nonref >= T - 64],
                                    rng.choice(nonref[nonref < T], 128, replace=False)]))
    worst = 0.0
    for st in (0, 1):
        for h in (1, 6):
            worst = max(worst, check_compress_unit(shape, xs[st][0, h], caches[st], 0, h,
                                                   oracle_mlp(comps[st], dk.ACT_GELU), pos,
                                                   TOL[dk.BF16]))
    say(f"[case] stream-s8k8: sampled latent rel err {worst:.3e}")
    kdw = xavier_mlp(w.d_c, w.hidden, d, key=(2, widx, 0, 0), dtype=torch.bfloat16)
    vdw = xavier_mlp(w.d_c, w.hidden, d, key=(2, widx, 0, 1), dtype=torch.bfloat16)
    q = queries(H * G, d, key=(3, widx), dtype=torch.bfloat16).reshape(B, H * G, d)
    scale = 1.0 / math.sqrt(d)
    out = gpu_decode(shape, H * G, cap, q, caches[0], gpu_mlp(kdw, dk.ACT_GELU), caches[1],
                     gpu_mlp(vdw, dk.ACT_GELU), scale)
    h = 5
    want = oracle_decode_head(shape, cap, to_np(q[0, h * G:(h + 1) * G]), caches[0], caches[1],
                              0, h, oracle_mlp(kdw, dk.ACT_GELU), oracle_mlp(vdw, dk.ACT_GELU),
                              scale)
    err = rel_err_rows(out[0, h * G:(h + 1) * G], want)
    say(f"[case] stream-s8k8: decode rel err {err:.3e} (KV head {h})")
    assert err <= TOL[dk.BF16]


def test_batch8_llama_layer_128k_sampled():
    # one layer of the batch-8 128k workload (8 sequences x 8 KV heads = 64
    # units per stream, per-sequence seeds): one compress call per stream over
    # every sequence's whole prefix and one decode call; the oracle checks
    # sampled tokens of units in the first and last sequence and the decode of
    # one KV head of sequence 6 over all 131072 positions
    from deltakv_synth import WORKLOADS, workload_index, unit_key
    w = WORKLOADS["llama8b-32layer-T128k-batch8-bf16"]
    widx = workload_index(w.name)
    B, H, G, T, d, s = w.batch, w.kv_heads, w.q_heads // w.kv_heads, w.T, w.head_dim, w.stride
    shape = dk.Shape(B, H, d, s, w.k, w.d_c, T, dk.BF16)
    say("[case] batch8-T128k one layer: generating and compressing on the GPU")
    xs, caches, comps = [], [], []
    for st in (0, 1):
        x = torch.empty(B, H, T, d, dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            for h in range(H):
                x[b, h] = kv_rows(T, d, w.n_dirs, w.n_centroids, key=unit_key(widx, b, 0, h, st),
                                  dtype=torch.bfloat16, device="cuda")
        cw = xavier_mlp(d, w.hidden, w.d_c, key=(1, widx, 0, st), dtype=torch.bfloat16)
        cache = dk.Cache(shape)
        dk.build_refs(shape, x, 0, T, cache)
        ws = dk.workspace(dk.compress_workspace_bytes(shape, 0, T))
        dk.compress(shape, x, 0, T, gpu_mlp(cw, dk.ACT_GELU), cache, ws)
        torch.cuda.synchronize()
        xs.append(x[[0, B - 1]].cpu())   # the sequences the oracle checks
        caches.append(cache)
        comps.append(cw)
        del x, ws
    nonref = oracle.nonref_positions(T, s)
    rng = np.random.default_rng(13)
    pos = np.unique(np.concatenate([nonref[:32], nonref[-32:],
                                    rng.choice(nonref, 64, replace=False)]))
    worst = 0.0
    for st in (0, 1):
        for i, (b, h) in enumerate([(0, 2), (B - 1, 5)]):
            worst = max(worst, check_compress_unit(shape, xs[st][i, h], caches[st], b, h,
                                                   oracle_mlp(comps[st], dk.ACT_GELU), pos,
                                                   TOL[dk.BF16]))
    say(f"[case] batch8-T128k: sampled latent rel err {worst:.3e}")
    kdw = xavier_mlp(w.d_c, w.hidden, d, key=(2, widx, 0, 0), dtype=torch.bfloat16)
    vdw = xavier_mlp(w.d_c, w.hidden, d, key=(2, widx, 0, 1), dtype=torch.bfloat16)
    q = queries(B * H * G, d, key=(3, widx), dtype=torch.bfloat16).reshape(B, H * G, d)
    scale = 1.0 / math.sqrt(d)
    out = gpu_decode(shape, H * G, T, q, caches[0], gpu_mlp(kdw, dk.ACT_GELU), caches[1],
                     gpu_mlp(vdw, dk.ACT_GELU), scale)
    b, h = 6, 1
    want = oracle_decode_head(shape, T, to_np(q[b, h * G:(h + 1) * G]), caches[0], caches[1], b,
                              h, oracle_mlp(kdw, dk.ACT_GELU), oracle_mlp(vdw, dk.ACT_GELU), scale)
    err = rel_err_rows(out[b, h * G:(h + 1) * G], want)
    say(f"[case] batch8-T128k: decode rel err {err:.3e} (sequence {b}, KV head {h})")
    assert err <= TOL[dk.BF16]
