"""The benchmark's byte model (the algorithmic bytes behind roofline.achieved
and value) on small workloads, against counts made independently here, and
the one-GPU guard of bench.py (CPU only)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_case, make_fork_case, make_prefix_case, make_private_case  # noqa: E402


def _slots_by_set(case):
    """Distinct (physical block, offset) pairs read, with a Python set."""
    seen = set()
    for s, L in enumerate(case.context_lens.tolist()):
        for t in range(L):
            seen.add((int(case.block_tables[s, t // case.block_size]), t % case.block_size))
    return len(seen)


def test_unique_slots_counts_shared_blocks_once():
    c = make_prefix_case("acct-prefix", [3, 40, 70, 100, 33, 64, 90, 17], 4, 32, 8, 2, 64, 16,
                         "bf16", 1)
    assert bench.unique_slots(c) == _slots_by_set(c)
    assert bench.unique_slots(c) < int(c.context_lens.sum())
    f = make_fork_case("acct-fork", [50, 50, 50, 50, 20, 90], 1, 4, 8, 2, 64, 16, "bf16", 2)
    assert bench.unique_slots(f) == _slots_by_set(f)
    p = make_private_case("acct-private", [1, 16, 17, 100], 8, 2, 64, 16, "bf16", 3)
    assert bench.unique_slots(p) == int(p.context_lens.sum())


def test_decode_bytes_of_the_tiny_fp32_workload():
    """Config 0: lengths 1, 17, 33, 100 (151 tokens), 2 KV heads of 64 fp32
    elements: K and V rows 2 * 151 * 2 * 64 * 4 = 154,624 bytes; q (fp32) and
    out (fp32) 4 * 2 * 64 * 8 = 4,096; used table entries 1 + 2 + 3 + 7 = 13
    of 4 bytes and 4 lengths, 68; one partition, no dispatch list."""
    c = make_case(0)
    assert int(c.context_lens.sum()) == 151
    assert bench.decode_bytes(c, 1, 0, unique=False) == 154_624 + 4_096 + 68
    assert bench.decode_bytes(c, 1, 0, unique=True) == 154_624 + 4_096 + 68


def test_decode_bytes_counts_split_partials():
    """Split sequences add their per-partition partials, written by decode and
    read by the merge: 2 * partitions * Hq * (D + 2) * 4 bytes each."""
    c = make_private_case("acct-split", [100, 300, 64], 8, 2, 64, 16, "bf16", 4)
    one = bench.decode_bytes(c, 1, 0, unique=False)
    split = bench.decode_bytes(c, 5, 64, unique=False)
    # 100 tokens -> 2 partitions of 64, 300 -> 5, 64 -> 1 (not split)
    assert split - one == 2 * (2 + 5) * 8 * (64 + 2) * 4


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_option_guards():
    """The 8-bit options reach their own entry points in both modes: the
    multi-query mode picks the FP8 or INT8 multi-query call, the decode mode
    the FP8 or INT8 decode (no multi-query guard in the decode path)."""
    src = open(os.path.join(ROOT, "bench.py")).read()
    body = src[src.index("def multi_query_bench"):src.index("def main")]
    assert "pa.paged_attention_multi_query_fp8 if args.kv_fp8 else" in body
    assert "pa.paged_attention_multi_query_int8" in body
    main = src[src.index("def main"):]
    assert "pa.paged_attention_decode_fp8 if args.kv_fp8 else pa.paged_attention_decode_int8" \
        in main
    assert "is not available with --multi-query" not in src
