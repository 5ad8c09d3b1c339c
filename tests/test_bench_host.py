"""Host-side logic of bench.py: the retrieve's algorithmic byte and flop counts, the rule that
keeps counter traffic only while it was measured on the current kernel source, and the refusal of
more than one GPU.  No GPU is touched."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_retrieve_bytes_of_the_8b3b_layer():
    # one 8B->3B layer at L = 32768 (32 sender heads, 24 query / 8 KV receiver heads, d = 128,
    # B = 64, 512 block rows) with the benchmark's mean kept-block count: 24.85 GB per launch, of
    # which the kept probabilities (256 KiB per block) are about 98%
    nnzb = 92967
    total = bench.retrieve_bytes(nnzb, 32, 64, 512, 32768, 8, 24, 128)
    assert abs(total - 24.85e9) < 0.01e9
    probs = nnzb * 256 * 1024
    assert 0.975 < probs / total < 0.985
    # every term scales as stated: one more kept block adds its probabilities and its index
    assert bench.retrieve_bytes(nnzb + 1, 32, 64, 512, 32768, 8, 24, 128) - total == 256 * 1024 + 4


def test_retrieve_flops_per_kept_block():
    # per kept block of the 8B->3B pair: 6.3 MFLOP of head mix plus 25.2 MFLOP of P.V
    per_block = bench.retrieve_flops(1, 32, 24, 64, 128)
    assert abs(per_block - 31.46e6) < 0.01e6
    mix = 2 * 24 * 32 * 64 * 64
    assert abs(mix - 6.29e6) < 0.01e6


def test_counter_traffic_needs_the_current_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "retrieve.hip"
    src.write_bytes(b"// kernel source\n")
    (tmp_path / "profiles").mkdir()
    rec = {"w": {"source_sha256": hashlib.sha256(src.read_bytes()).hexdigest(), "bytes_per_launch": 123.0}}
    (tmp_path / "profiles" / "retrieve_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile(str(src), "w") == 123.0
    assert bench.traffic_from_profile(str(src), "other") is None
    src.write_bytes(b"// kernel source, changed\n")
    assert bench.traffic_from_profile(str(src), "w") is None


def test_committed_counter_traffic_matches_the_committed_retrieve():
    # the benchmark reports counter traffic only while the summary was taken on this source
    with open(os.path.join(ROOT, "profiles", "retrieve_traffic.json")) as f:
        recs = json.load(f)
    for wl in ("full_8b3b_32k", "pair_8b3b_8k", "varlen_14b8b", "long_131k"):
        got = bench.traffic_from_profile(bench.RETRIEVE_SRC, wl)
        assert got is not None, f"{wl}: counter traffic taken on another retrieve source"
        assert got == recs[wl]["bytes_per_launch"]
        assert got >= recs[wl]["algorithmic_bytes_per_launch"]


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
