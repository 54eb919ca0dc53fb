"""CPU: the host side of bench.py -- its one-GPU contract, its workload table
and the recorded HBM traffic it reports (no GPU calls)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quant_integer_dot_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr


def test_extra_rows_of_the_default_line_can_be_skipped(monkeypatch):
    """The default decode line carries the shard rows and the M = 512 prefill
    row; profiling runs switch each off, and the defaults keep both on."""
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.workload == "qwen3-8b-decode" and not a.no_shard_rows and not a.no_prefill_row
    monkeypatch.setattr(sys, "argv", ["bench.py", "--no-shard-rows", "--no-prefill-row"])
    a = bench.parse()
    assert a.no_shard_rows and a.no_prefill_row


@pytest.mark.parametrize("name", ["qwen3-8b-decode", "qwen3-8b-prefill-512", "iq4xs-h5120-decode",
                                  "qwen2.5-1.5b-decode", "qwen3-8b-q4_0-q8_0-decode", "qwen3-8b-mid-batch",
                                  "qwen3-8b-tp8-shard-decode"])
def test_workloads_match_the_synthetic_configs(name):
    """Each bench workload has the shapes and layer count of the synthetic
    config it names, and M values inside that config's list."""
    cfg_idx, shapes, layers, Ms = bench.workload_def(name)
    w = synth.WORKLOADS[cfg_idx]
    assert w["name"] == name
    assert shapes == w["shapes"] and layers == w["layers"]
    assert set(Ms) <= set(w["Ms"])


def test_tp8_shard_shapes():
    """The tensor-parallel share: q, k, v, gate, up split by rows, o and down
    by K, 8 ways, on superblock boundaries; together an eighth of the
    layer's weights."""
    full = {n: (N, K, t) for n, N, K, t in synth.QWEN3_8B}
    for n, N, K, t in synth.QWEN3_8B_TP8:
        fN, fK, ft = full[n]
        assert t == ft
        if n in ("o", "down"):
            assert (N, K * 8) == (fN, fK) and K % 256 == 0
        else:
            assert (N * 8, K) == (fN, fK)
    wb = lambda shapes: sum(synth.weight_bytes(t, N, K) for _, N, K, t in shapes)
    assert wb(synth.QWEN3_8B_TP8) * 8 == wb(synth.QWEN3_8B)
    assert [s for s in synth.QWEN3_8B_TP8 if s[0] in ("gate", "up", "down")] == bench.shard_rows_shapes()


def test_c0_workload_is_cold():
    """C0 runs the single 1536 x 1536 Q4_K matrix as distinct copies whose
    total is over twice the 256 MB Infinity Cache."""
    cfg_idx, shapes, layers, Ms = bench.workload_def("q4k-matvec-1536")
    assert cfg_idx == 0 and shapes == synth.WORKLOADS[0]["shapes"] and Ms == [1]
    name, N, K, t = shapes[0]
    assert layers * synth.weight_bytes(t, N, K) > 2 * 256e6


@pytest.mark.parametrize("kernel,workload", [("qmv_multi_kernel", "qwen3-8b-decode"),
                                             ("qmm_mfma_kernel", "qwen3-8b-prefill-512"),
                                             ("qmm_skinny_kernel", "qwen3-8b-mid-batch"),
                                             ("rmsnorm_q8_1_kernel", "qwen3-8b-rmsnorm-q8_1"),
                                             ("attn_kv4_partial_kernel+attn_kv4_combine_kernel",
                                              "qwen3-8b-attn-kv4-32k")])
def test_recorded_traffic_matches_the_sources(kernel, workload):
    """Each measured kernel has a committed HBM-traffic summary, and the bench
    line reports its figure only while the summary's source digest matches
    the current kernel sources (null once a kernel has changed since the
    counters were taken)."""
    import glob
    found = None
    for path in glob.glob(os.path.join(bench.ROOT, "profiles", "hbm_traffic_*.md")):
        text = open(path).read()
        if f"kernel: {kernel}\n" in text and f"workload: {workload}\n" in text:
            found = text
    assert found is not None, (kernel, workload)
    kv = dict(line.split(": ", 1) for line in found.splitlines()
              if ": " in line and not line.startswith(("|", "#", " ")))
    assert int(kv["traffic_bytes_per_launch"]) > 0
    current = bench.kernel_source_digest(kv["source_files"].split()) == kv["source_digest"]
    t = bench.recorded_traffic(kernel, workload)
    assert (t == int(kv["traffic_bytes_per_launch"])) if current else (t is None)
