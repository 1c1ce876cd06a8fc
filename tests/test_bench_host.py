"""Host checks of bench.py's reporting (no GPU): the metric's FLOP count,
the refusal of multi-GPU runs, and the rule that a committed counter
summary only counts while its kernel's sources are unchanged."""
import json
import os
import shutil

import pytest

import bench
from test_weight_mlp_amd import inputs

T, D, F, C = 32768, 2560, 9728, 512          # the default workload: 4B shape, 32k tokens
N = T // C
MAIN = 8 * T * D * F                          # Z (4 Tdf), the chunk deltas (2 Tdf), the apply (2 Tdf)
TARGET = 2 * T * D * D + 10 * T * D           # W_target (2 d^2) and the five-tap Conv1D (10 d) per token
ADDS = N * D * F                              # one d x f state add per chunk
LAST = 2 * C * D * F                          # the last chunk's delta


def test_default_workload_flops():
    cfg = inputs.CONFIGS["4b_32k"]
    assert (cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk) == (1, T, D, F, C)
    assert bench.algorithmic_flops(cfg) == MAIN + TARGET + ADDS - LAST == 6_934_778_347_520


def test_flop_variants():
    cfg = inputs.CONFIGS["4b_32k"]
    base = MAIN + ADDS - LAST
    assert bench.algorithmic_flops(cfg, "no_conv") == base + 2 * T * D * D
    assert bench.algorithmic_flops(cfg, "no_proj") == base + 10 * T * D
    # a carried-out state needs the last chunk's delta too
    assert bench.algorithmic_flops(cfg, carry=True) == MAIN + TARGET + ADDS
    # a training step counts three forwards
    assert bench.algorithmic_flops(cfg, backward=True) == 3 * (MAIN + TARGET + ADDS - LAST)
    # a ragged last chunk: 1000 tokens in chunks of 256 leave 232 in the last
    small = cfg.with_(seq_len=1000, chunk=256, d_model=64, d_ff=128)
    assert small.n_chunks == 4
    assert bench.algorithmic_flops(small, "no_proj") == (8 * 1000 * 64 * 128 + 10 * 1000 * 64 + 4 * 64 * 128
                                                         - 2 * 232 * 64 * 128)


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
    monkeypatch.setenv("WORLD_SIZE", "2")
    assert bench.main([]) == 2


def test_counter_summary_counts_only_for_unchanged_sources(tmp_path, monkeypatch):
    kernel = "scan_fast_kernel"
    src = os.path.join(bench.ROOT, "test_weight_mlp_amd", "csrc")
    os.makedirs(tmp_path / "test_weight_mlp_amd" / "csrc")
    for f in bench.KERNEL_SOURCES[kernel]:
        shutil.copy(os.path.join(src, f), tmp_path / "test_weight_mlp_amd" / "csrc" / f)
    os.makedirs(tmp_path / "profiles")
    summary = {"kernel": kernel, "source_sha": "", "bytes_per_launch": 123.0}
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    summary["source_sha"] = bench.source_sha(kernel)
    (tmp_path / "profiles" / f"{kernel}_traffic.json").write_text(json.dumps(summary))
    assert bench.traffic_from_profile(kernel) == 123.0
    # any edit to one of the kernel's sources retires the summary
    with open(tmp_path / "test_weight_mlp_amd" / "csrc" / bench.KERNEL_SOURCES[kernel][0], "a") as fh:
        fh.write("\n")
    assert bench.profile_of(kernel) == {}
    assert bench.traffic_from_profile(kernel) is None


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_committed_summaries_name_their_kernel_and_workload(kernel):
    path = os.path.join(bench.ROOT, "profiles", f"{kernel}_traffic.json")
    with open(path) as fh:
        t = json.load(fh)
    assert t["kernel"] == kernel and t["workload"] == "4b_32k"
    assert t["bytes_per_launch"] == pytest.approx(t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"])
