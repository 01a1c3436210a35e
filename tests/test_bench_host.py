"""bench.py's host-side contract (no GPU): one GPU only, and the byte counts
the line divides by."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_match_the_layout(orc):
    """group_bytes: reduce = 2 L valid + 4 N S, placement = 4 valid, for the
    headline group, with S from the oracle's layout."""
    sys.path.insert(0, ROOT)
    import bench
    from workloads.configs import CONFIGS
    cfg = CONFIGS["padding_stress"]
    S = int(orc.layout(cfg.shapes, cfg.N)["S"])
    rs, ag, valid = bench.group_bytes(cfg, S)
    assert valid == sum(t * k for t, k in cfg.shapes) == 1961576166
    assert S == 41196789
    assert rs == 2 * cfg.L * valid + 4 * cfg.N * S
    assert ag == 4 * valid
    assert rs + ag == 47141306808
