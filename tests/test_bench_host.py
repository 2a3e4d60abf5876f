"""Host logic of bench.py, no GPU: the one-GPU guard, the counter readings' source hashes, and the
algorithmic units the roofline figures divide by (each against the count written out by hand)."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gated_deltanet_delta_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""          # no JSON line for a configuration that was not measured


@pytest.mark.parametrize("kernel", sorted(bench.COUNTERS))
def test_counter_readings_match_their_sources(kernel):
    """Every committed counter reading names the source it was taken at; a stale one would make
    the bench report null traffic, so the hashes must follow the sources."""
    c = bench.COUNTERS[kernel]
    assert os.path.isfile(os.path.join(ROOT, c["source"]))
    assert c["sha16"] == bench.source_sha16(c["source"]), f"{kernel}: counters predate {c['source']}"
    for key in c:
        if key not in ("source", "sha16"):
            assert bench.counter(kernel, key) == c[key]


def test_counter_is_null_for_a_changed_source(monkeypatch):
    monkeypatch.setitem(bench.COUNTERS, "scan", dict(bench.COUNTERS["scan"], sha16="0" * 16))
    assert bench.counter("scan", "traffic") is None
    assert bench.counter("decode", "missing-key") is None


def test_prefill_units():
    wl = synth.WORKLOADS["prefill"]
    nbytes, flops, per_tok_head = bench.prefill_algorithmic(wl, wl.T, wl.B, 1, False)
    # q, k: 128 bf16 each, shared by the two v-heads of a k-head; v: 128 bf16; g, beta: bf16;
    # o: 128 fp32
    assert per_tok_head == (128 * 2 + 128 * 2) / 2 + 128 * 2 + 2 * 2 + 128 * 4 == 1028
    state = 128 * 128 * 4
    assert nbytes == 4096 * 32 * 1028 + 32 * state          # final state only (zero initial)
    assert bench.prefill_algorithmic(wl, wl.T, wl.B, 1, True)[0] == nbytes + 32 * state
    # three 128 x 128 contractions per token, 2 flops per multiply-add; the intra-chunk products
    # over up to 64 positions: Q K^T and the two C x dv products with k/q
    assert flops == 4096 * 32 * 139264
    assert 6 * 128 * 128 + 64 * (3 * 128 + 2 * 128) == 139264


def test_decode_units():
    wl = synth.WORKLOADS["decode"]
    state, total = bench.decode_algorithmic(wl)
    assert state == 2 * 256 * 32 * 128 * 128 * 4 == 1073741824
    io = 256 * (2 * 16 * 128 * 2 + 32 * 128 * 2 + 2 * 32 * 4 + 32 * 128 * 4)
    assert total - state == io


def test_backward_flop_unit():
    # per 64-token chunk and v-head at dk = dv = 128: K K^T and Q K^T (lower halves), ten
    # dk x dv-sized products, six C x C x dv and three C x C x dk triangular products (halves)
    macs = 2 * (64 * 64 * 128 // 2) + 10 * 64 * 128 * 128 + 6 * (64 * 64 * 128 // 2) \
        + 3 * (64 * 64 * 128 // 2)
    assert 2 * macs // 64 == bench.BWD_FLOPS_PER_TOKEN_VHEAD == 417792
