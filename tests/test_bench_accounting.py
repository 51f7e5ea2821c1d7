"""The benchmark's algorithmic byte model against the per-block totals worked out
from the workload shapes (every touched BF16 weight once, the KV rows read and
written, the gathered embedding rows; MoE: only the experts the rows touch)."""
import importlib.util
import os

import pytest

from verifier_block_forward_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,total_mb,touched", [
    ("c1", 2612.8, None), ("c2", 3459.3, None), ("c3", 3114.8, None), ("c4", 1179.7, [8]),
])
def test_per_block_totals(bench, name, total_mb, touched):
    cfg = configs.get(name)
    b = bench.class_bytes(cfg, cfg.M, cfg.R, cfg.C, touched)
    assert abs(b["total"] / 1e6 - total_mb) < 0.15, b["total"]
    assert b["total"] == b["projections"] + b["attention"] + b["row_kernels"] + b["lm_head"]


def test_moe_bytes_count_touched_experts(bench):
    cfg = configs.get("c4m4")
    H, Ie = cfg.hidden, cfg.expert_intermediate
    lo = bench.class_bytes(cfg, cfg.M, 0, cfg.C, [8])
    hi = bench.class_bytes(cfg, cfg.M, 0, cfg.C, [31])
    assert hi["projections"] - lo["projections"] == 23 * 3 * Ie * H * 2
    # about 30.5 distinct experts for 4 rows x top-8 of 256 gives ~1321 MB per block
    mid = bench.class_bytes(cfg, cfg.M, 0, cfg.C, [30])["total"] / 1e6
    assert 1300 < mid < 1330


def test_lm_head_share_c1(bench):
    cfg = configs.get("c1")
    b = bench.class_bytes(cfg, cfg.M, cfg.R, cfg.C)
    assert b["lm_head"] == 262144 * 2816 * 2
    assert abs(b["lm_head"] / b["total"] - 0.565) < 0.001
