"""Host-side checks of the benchmark harness and the workload table (no GPU).

The workload parameters are the ones the benchmark and the parity tests run:
a tiny single-head fp32 case, one Llama-3.1-8B-shaped layer at 32k, the full
32-layer cache at 128k, the same at batch 8, and the streaming prompt with
references accumulating online (DeltaKV page, section 1 for the 128k / batch 8
setting, section 3 for stride, k and the Compressor / Decompressor widths).
"""
import os
import subprocess
import sys

from deltakv_synth import WORKLOADS, workload_index

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu_before_touching_a_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 2
    assert "one GPU only" in r.stdout
    assert "--gpus 2" in r.stdout


def test_workload_table_shapes():
    want = {
        "tiny-1head-T512-fp32": dict(layers=1, batch=1, kv_heads=1, q_heads=1, head_dim=64,
                                     T=512, stride=16, k=4, d_c=16, hidden=128, dtype="fp32",
                                     n_dirs=4, n_centroids=32, chunk=None, appends=0),
        "llama8b-1layer-T32k-bf16": dict(layers=1, batch=1, kv_heads=8, q_heads=32,
                                         head_dim=128, T=32768, stride=16, k=4, d_c=32,
                                         hidden=256, dtype="bf16", n_dirs=8,
                                         n_centroids=1024, decode_steps=256),
        "llama8b-32layer-T128k-bf16": dict(layers=32, batch=1, kv_heads=8, q_heads=32,
                                           head_dim=128, T=131072, stride=16, k=4, d_c=32,
                                           hidden=256, dtype="bf16", decode_steps=128),
        "llama8b-32layer-T128k-batch8-bf16": dict(layers=32, batch=8, T=131072, stride=16,
                                                  k=4, d_c=32, hidden=256, dtype="bf16"),
        "llama8b-32layer-T128k-stream-s8k8-bf16": dict(layers=32, batch=1, T=131072,
                                                       stride=8, k=8, d_c=16, hidden=256,
                                                       dtype="bf16", chunk=4096,
                                                       appends=1024, decode_steps=1024),
    }
    assert list(WORKLOADS) == list(want)
    for name, fields in want.items():
        wl = WORKLOADS[name]
        assert wl.name == name
        for f, v in fields.items():
            assert getattr(wl, f) == v, (name, f)
        assert workload_index(name) == list(want).index(name)
    # grouped-query attention: whole groups of query heads per KV head
    for wl in WORKLOADS.values():
        assert wl.q_heads % wl.kv_heads == 0
    # the 128k batch-8 cache uncompressed: 137.44 GB (more than 130 GB)
    b8 = WORKLOADS["llama8b-32layer-T128k-batch8-bf16"]
    full = b8.batch * b8.T * b8.layers * b8.kv_heads * b8.head_dim * 2 * 2
    assert full == 137_438_953_472
