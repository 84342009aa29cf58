"""Host checks of bench.py's contract (CPU only): more than one GPU is refused
with a message, no GPU is refused, the block-sparse workload's selection and
pair count are what the bench line states, and the HBM-traffic lookup only
accepts counter summaries taken on the current kernel source."""
import json
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from differential_attention_02_amd import workloads  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_no_gpu_is_refused():
    if torch.cuda.is_available():
        return
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "no GPU" in r.stderr


def test_sparse_selection_shape_budget_and_pairs():
    cfg = workloads.CONFIGS["v2_prefill_4k"]
    mask, pairs = bench._sparse_selection(cfg)
    assert tuple(mask.shape) == (cfg.batch, cfg.q_heads // 2, 32, 64)
    per_tile = mask.sum(-1)
    # query tile t sees key tiles 0 .. 2t + 1 (causal); the budget is 16
    expect = torch.clamp(2 * torch.arange(32) + 2, max=16)
    assert torch.equal(per_tile, expect.expand_as(per_tile))
    assert bool(mask[..., 0].all())                         # the first key tile is always kept
    t = torch.arange(32)
    for back in range(4):                                   # the four tiles ending at the query tile's last row
        tt = t[2 * t + 1 - back >= 0]
        assert bool(mask[:, :, tt, 2 * tt + 1 - back].all())
    assert not bool(mask[:, :, t[:-1], (2 * t + 2)[:-1]].any())   # nothing past the causal limit
    # pairs: brute force over one (batch, pair) slice equals the closed-form count
    one = workloads.block_pairs(mask[:1, :1], cfg.seqlen)
    m = mask[0, 0]
    rows = torch.arange(cfg.seqlen)
    allowed = m[rows[:, None] // 128, rows[None, :] // 64] & (rows[None, :] <= rows[:, None])
    assert one == int(allowed.sum())
    assert 0.40 < pairs / (cfg.batch * (cfg.q_heads // 2) * cfg.pairs) < 0.43


def test_traffic_lookup_requires_current_source(tmp_path, monkeypatch):
    rec = {"hbm_bytes_per_launch": 123.0, "source_digest": bench._kernel_digest(bench.V2P_SOURCES)}
    (tmp_path / "good.md").write_text("x\ntraffic_json: " + json.dumps(rec) + "\n")
    rec["source_digest"] = "0" * 16
    (tmp_path / "stale.md").write_text("traffic_json: " + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench._traffic_from_profile("good.md", bench.V2P_SOURCES) == 123.0
    assert bench._traffic_from_profile("stale.md", bench.V2P_SOURCES) is None
    assert bench._traffic_from_profile("missing.md", bench.V2P_SOURCES) is None
