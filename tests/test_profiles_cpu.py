"""The committed profile summaries match the code they describe: the HBM
counter summary of the scoring kernel was taken on the current source of
that kernel (else bench.py would report its traffic as unknown), and every
summary names the command that produced it."""
import glob
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_score_counters_match_current_source():
    traffic = bench._counter_traffic("score", bench.SCORE_SOURCES, "llama7b_32k_layer")
    assert traffic is not None, "re-take the scoring kernel's FETCH_SIZE / WRITE_SIZE counters"
    # keys (268435456 B) + logits (8388608 B) + the 1 MiB prefetch read and written
    algorithmic = 268435456 + 8388608 + 2 * 1048576
    assert abs(traffic - algorithmic) <= 0.01 * algorithmic


def test_every_profile_names_its_command():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt")))
    assert files
    for path in files:
        with open(path) as f:
            text = f.read()
        assert "rocprofv3" in text, path
        assert "bench.py" in text, path
