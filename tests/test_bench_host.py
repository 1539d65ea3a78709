"""Host-side checks of bench.py that need no GPU: the algorithmic byte and
flop counts against a hand count, the traffic records it reads, and the
one-GPU contract of its command line."""
import os
import subprocess
import sys

import numpy as np

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_step_traffic_hand_count():
    # tiny fp32 layer: H 256, 8 experts top-2, I 512, one shared expert of 512
    cfg = W.CONFIGS["tiny"]
    H, E, I, Is = 256, 8, 512, 512
    assert (cfg.hidden, cfg.n_experts, cfg.inter, cfg.shared_inter, cfg.n_shared) == (H, E, I, Is, 1)
    ids = np.array([[0, 1], [0, 2]])
    exact = np.array([[1, 1], [1, 0]], dtype=np.uint8)   # expert 2 left to the surrogate
    tr = bench.step_traffic(cfg, 2, "lore", ids, exact)
    r = cfg.lore_rank
    by = (H * E * 4 + 2 * 2 * H * 4          # router weights, x in and out
          + 2 * 3 * I * H * 4                # experts 0 and 1, gate/up/down
          + 3 * Is * H * 4                   # shared expert
          + 1 * 2 * r * H * 4)               # LoRE A and B of expert 2
    fl = 2 * 2 * H * E + 3 * 2 * 3 * I * H + 2 * 2 * 3 * Is * H + 1 * 2 * 2 * r * H
    assert tr["bytes"] == by
    assert tr["flops"] == fl
    assert (tr["distinct_experts"], tr["lore_experts"], tr["pairs"]) == (2, 1, 3)
    up = tr["up"]
    assert up["bytes"] == ((2 * 2 * I * H + 2 * Is * H + 1 * r * H) * 4 + 2 * H * 4
                           + (3 * I + 2 * Is + 1 * r) * 4)
    assert up["flops"] == 3 * 2 * 2 * I * H + 2 * 2 * 2 * Is * H + 1 * 2 * r * H


def test_traffic_records_parse_and_name_existing_sources():
    assert bench.TRAFFIC_FILES
    for key, path in bench.TRAFFIC_FILES.items():
        rec = bench.recorded_traffic(path)
        assert rec is not None, path
        nbytes, srcs, digest = rec
        assert nbytes > 0 and len(digest) == 16
        for s in srcs:
            assert os.path.exists(os.path.join(ROOT, s)), s


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
