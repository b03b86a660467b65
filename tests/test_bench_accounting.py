"""bench.py's algorithmic work per launch: the byte and flop counts its
roofline fractions divide by, for every workload, against the hot-path
table's figures (norms: read x once and write L rows, plus the weights;
store: one shared slot mapping, each row's position with RoPE, cos/sin and
K/V of the rows with a slot; projection: 2 L T D N)."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

TABLE = {  # workload: (norm bytes, store bytes, projection flop)
    "tiny": (835_584, 16_384, 6.71e7),
    "prefill": (42_024_960, 8_033_024, 3.436e10),
    "weightless": (335_609_856, 67_141_632, 2.749e11),
    "long": (1_342_259_200, 270_794_752, 1.0995e12),
    "edge": (4_831_985_664, 1_076_363_264, 8.796e12),
}


@pytest.mark.parametrize("name", sorted(TABLE))
def test_algorithmic_work_matches_the_table(name):
    sys.path.insert(0, ROOT)
    import bench
    from norm_rope_cache_amd import synth

    cfg = synth.CONFIGS[name]
    norms, store, flops = bench.algorithmic_bytes(cfg, synth.slot_mapping(cfg))
    want_n, want_s, want_f = TABLE[name]
    assert norms == want_n
    assert store == want_s
    assert abs(flops - want_f) <= 5e-4 * want_f


def test_cpu_threads_respect_the_omp_cap(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    n, model = bench.host_cpu()
    assert 1 <= n <= 3 and isinstance(model, str) and model
