"""Host-side checks of bench.py that need no GPU: the one-GPU refusal, the
byte count the decode rooflines are priced with, and the traffic records."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("dead", [0, 37])
def test_expert_bytes_add_up_to_the_stored_tensor(bench, dead):
    """Summed over the experts, the per-expert byte count is every stored
    code word, scale and row-map entry of the tensor."""
    T = synth.make_tensor(3, 1, rows=96, cols=320, d=4, bits=11, n_experts=5, dead_rows=dead)
    total = T.codes.nbytes + T.scales.nbytes + (0 if T.row_map is None else T.row_map.nbytes)
    assert sum(bench.expert_bytes(T, e) for e in range(T.n_experts)) == total


def test_traffic_records_are_well_formed(bench):
    """Each record names a known workload, a 16-hex-digit source hash and a
    positive byte count."""
    known = set(synth.WORKLOADS) | set(synth.STACK_WORKLOADS) | set(synth.GATHER_WORKLOADS) \
        | set(synth.FIT_WORKLOADS)
    with open(bench.TRAFFIC) as f:
        lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert lines
    for ln in lines:
        assert ln[0] in known, ln[0]
        assert len(ln[1]) == 16 and int(ln[1], 16) >= 0
        assert int(ln[2]) > 0


def test_source_hash_tracks_the_family_files(bench):
    h = {f: bench.kernel_source_hash(f) for f in ("decode", "prefill", "gather", "fit")}
    assert len(set(h.values())) == 4
    assert all(len(v) == 16 for v in h.values())
