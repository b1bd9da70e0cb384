"""Host-side checks of bench.py that need no GPU: it refuses more than one GPU
before touching one, the algorithmic byte and flop counts behind its roofline
figures agree with counts taken a different way (from the arrays' own sizes and
a per-head, per-position tally), and the traffic reader only accepts a counter
summary taken on the current kernel source."""
import os
import re
import subprocess
import sys

import pytest

import bench
from workloads import MINI, TINY, all_workloads, make_attn_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line for a refused run


@pytest.mark.parametrize("name", ["tiny", "mini_gqa8_d15", "mini_fp8_d15", "mini_hd64_g4"])
def test_algorithmic_bytes_from_array_sizes(name):
    w = TINY if name == "tiny" else MINI[name]
    inp = make_attn_inputs(w)
    L = [int(x) for x in inp.kv_lens]
    # one (block, KV head) image of K holds 16 keys; V has the same size
    per_key = inp.k_cache[0, 0].nbytes // 16
    kv = sum(L) * inp.k_cache.shape[1] * per_key * 2
    blocks = sum(-(-x // 16) for x in L)
    table = blocks * inp.block_table.itemsize
    scales = 0 if inp.k_scale is None else blocks * inp.k_scale.shape[1] * inp.k_scale.itemsize * 2
    q_and_out = 2 * inp.q.nbytes
    assert bench.attn_algorithmic_bytes(inp) == kv + table + scales + q_and_out
    assert bench.attn_algorithmic_kv_bytes(inp) == kv


@pytest.mark.parametrize("name", ["tiny", "mini_gqa8_d15", "mini_mqa_d3"])
def test_algorithmic_flops_by_query_head_and_position(name):
    w = TINY if name == "tiny" else MINI[name]
    inp = make_attn_inputs(w)
    # every (query head, new position) row against every key of its sequence:
    # a q.k dot product and a p.v accumulation, 2 hd flops each
    flops = 0
    for b in range(w.B):
        for _h in range(w.H_q):
            for _i in range(w.R):
                flops += int(inp.kv_lens[b]) * 4 * w.hd
    assert bench.attn_algorithmic_flops(inp) == flops


def test_traffic_reader_matches_only_its_own_source():
    txt = open(bench.TRAFFIC_FILE).read()
    m = re.search(r"src_sha=(\w+)\s+workload=(\S+)\s+bytes_per_launch=(\d+)", txt)
    assert m, "the traffic summary carries its source hash, workload and bytes"
    got = bench.read_traffic(m.group(1))
    assert got == {"workload": m.group(2), "bytes": int(m.group(3))}
    assert bench.read_traffic("0" * 16) is None
    assert got["workload"] in all_workloads() and got["bytes"] > 0
