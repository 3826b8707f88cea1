"""CPU checks of bench.py's contract that need no GPU: a multi-GPU request is
refused with a message (this library measures one GPU), and the roofline's
`traffic` figure comes from a committed rocprofv3 counter summary only while
that summary's source hash matches the current kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

# (counter file's kernel, workload, kernel sources hashed)
ROOFLINE_COUNTERS = [("softmax_masked", "long", ("softmax_masked.hip", "common.hpp")),
                     ("softmax_masked", "prefill", ("softmax_masked.hip", "common.hpp")),
                     ("softmax_masked", "degen_sm", ("softmax_masked.hip", "common.hpp")),
                     ("decode_attn", "decode", ("decode.hip", "common.hpp")),
                     ("gdn_chain", "degen_lin", ("gdn.hip", "common.hpp"))]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr
    assert not any(line.startswith("{") for line in r.stdout.splitlines())


@pytest.mark.parametrize("kernel,workload,srcs", ROOFLINE_COUNTERS)
def test_traffic_only_for_matching_sources(kernel, workload, srcs):
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    with open(p) as f:
        c = json.load(f)
    h = bench.source_hash(*srcs)
    got = bench.counters_traffic(kernel, workload, h)
    # the committed summary either matches the sources (bytes reported) or is
    # stale (None): never a figure for a kernel that has changed since
    if c["source_hash"] == h:
        assert got == c["hbm_bytes_per_launch"] and got > 0
    else:
        assert got is None
    assert bench.counters_traffic(kernel, workload, "0" * 16) is None
    assert bench.counters_traffic(kernel, "no_such_workload", h) is None
