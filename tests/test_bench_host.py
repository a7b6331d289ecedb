"""bench.py on the host: the algorithmic work its rates divide by, and its one-GPU rule.

The counts are pinned to values derived by hand from the definitions (sums split
into the rows before and after the selection budget is reached, written as
exact integers), and on the 1K workload to a count of the oracle's own token
sets, so a wrong term in bench.py's vectorised formulas shows up here.
"""
import os
import subprocess
import sys

import numpy as np

import bench
import synth
from oracle import msa_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_32k_work_closed_form():
    s = synth.WORKLOADS[3]
    fm, fi, _ = bench.algorithmic_work(s)
    # rows t < 15 * 128 attend t + 1 keys; later rows 15 full blocks + (t mod 128) + 1
    early = 1920 * 1921 // 2
    late_rows = 32768 - 1920
    late = late_rows * 1921 + (late_rows // 128) * (127 * 128 // 2)
    assert fm == 4 * 128 * 64 * 2 * (early + late)
    # every row scores the 128 keys of each full block before its own
    keys = 128 * 128 * (255 * 256 // 2)
    assert fi == 2 * 128 * 4 * 2 * keys


def test_decode_128k_bytes_closed_form():
    for wid, c in ((4, 2), (6, 1)):
        s = synth.WORKLOADS[wid]
        _, _, by = bench.algorithmic_work(s)
        per_seq = (131072 * 128 * c            # the whole k_idx cache
                   + 4 * 16 * 128 * 128 * c * 2  # K and V of 16 blocks per group
                   + 2 * 64 * 128 * 2          # q in, out back
                   + 4 * 128 * 2               # q_idx
                   + 4 * 4 * 16)               # sel
        assert by == 64 * per_seq


def test_paged_bytes_reduce_to_the_decode_formula():
    s = synth.WORKLOADS[4]
    assert bench.paged_decode_bytes(s, [s.kv_len] * s.batch) == bench.algorithmic_work(s)[2]


def test_main_flops_count_the_oracle_token_sets():
    # 1K workload: 4 * d * Hq * (sum over rows of |T|), |T| from the oracle's selection
    s = synth.WORKLOADS[1]
    x = synth.host_inputs(s, 1)
    sel = orc.index_select(synth.as_f64(x["q_idx"]), synth.as_f64(x["k_idx"]), s.topk, s.q_offset)
    n_tok = 0
    n_keys = 0
    for i in range(s.q_len):
        t = s.q_offset + i
        n_tok += len(orc.token_set(sel[0, 0, i], t, s.block_size))
        n_keys += (t // s.block_size) * s.block_size
    fm, fi, _ = bench.algorithmic_work(s)
    assert fm == 4 * s.head_dim * s.num_q_heads * s.batch * n_tok
    assert fi == 2 * s.index_dim * s.groups * s.batch * n_keys


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == ""  # no JSON line


def test_main_branch_bytes_by_hand():
    # B=1, S_q=3, G=2, k=2, r=4, d=64, bf16; 128-token blocks over 300 keys (3 blocks)
    s = synth.Shape(1, 3, 300, 297, 8, 2, 64, 32, 2, dtype="bf16")
    import torch
    sel = torch.tensor([[[[0, 2], [1, -1], [2, -1]],
                         [[2, -1], [0, 1], [-1, -1]]]], dtype=torch.int32)
    m = bench.main_branch_bytes(s, sel)
    edges = 4 + 3                   # entries naming a block (group 0: 4, group 1: 3)
    buckets = 3 + 3                 # group 0 uses blocks {0, 1, 2}, group 1 uses {0, 1, 2}
    r, d = 4, 64
    assert m["edges"] == edges and m["buckets"] == buckets
    want = (edges * r * d * 2              # queries gathered
            + 2 * edges * r * (d * 2 + 4)  # partial states written and read back
            + buckets * 2 * 128 * d * 2    # K and V of every used block once
            + 2 * (1 * 2 * 3 * 2) * 4 + 2 * edges * 4  # selection read twice, entries written and read
            + 1 * 3 * 8 * (d * 2 + 4))     # output and lse
    assert m["total"] == want
    assert sum(m["parts"].values()) == want
