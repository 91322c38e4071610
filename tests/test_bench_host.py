"""Host-side accounting of bench.py, checked against the oracle's own partition and key sets
(CPU only): the flop count, the sparse key-set sizes, the merge's byte count, the traffic
record lookup and the single-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import helpers as hp
from context_mla_prefill_amd import synth
from oracle import attention as oa
from oracle import partition as op

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("cfg", [1, 2, 5, 6])
def test_attn_flops_counts_every_causal_pair(cfg):
    """The flops bench.py divides by: one multiply-add pair per latent+rope dim of Q K^T and
    per value dim of P V, for every (query, head, key) pair the causal rule admits: per rank
    launch of the oracle's partition, and for the step with every token once."""
    w = synth.workload(cfg)
    plan = hp.oracle_plan(w)
    per_flop = 2.0 * (w.Dl + w.Dr + w.Dl) * w.H
    for r in range(w.P):  # one rank's launch
        assert bench.attn_flops(plan.ranks[r].positions, w.H, w.Dl, w.Dr) == per_flop * op.causal_pairs(plan, r)
    # the step's value: every global token once equals the single-device causal count of
    # every request; the ranks together also compute the replicated rows P - 1 more times
    pos, _ = hp.token_maps(plan)
    whole = sum(int(kv) * (int(kv) + 1) // 2 - (int(kv) - int(q)) * (int(kv) - int(q) + 1) // 2
                for q, kv in zip(w.q_lens.tolist(), w.kv_lens.tolist()))
    assert bench.attn_flops(pos, w.H, w.Dl, w.Dr) == per_flop * whole
    repl = w.q_lens < 2 * w.P
    extra = sum(int(kv) * (int(kv) + 1) // 2 - (int(kv) - int(q)) * (int(kv) - int(q) + 1) // 2
                for q, kv in zip(w.q_lens[repl].tolist(), w.kv_lens[repl].tolist()))
    assert sum(op.causal_pairs(plan, r) for r in range(w.P)) == whole + (w.P - 1) * extra


def test_sparse_set_sizes_match_oracle_key_sets():
    """Random selected rows with pads, indices past the position, inside the window and
    duplicates of window keys: the sizes equal the oracle's key sets."""
    rng = np.random.default_rng(3)
    w = synth.custom(77, [300, 129, 1], [900, 129, 64], P=2, H=16, Dl=512, Dr=64, topk=48, window=16)
    plan = hp.oracle_plan(w)
    pos, _ = hp.token_maps(plan)
    rows = rng.integers(-1, 1000, size=(w.T_glob, w.topk)).astype(np.int32)
    rows = np.sort(rows, axis=1)
    for t in range(w.T_glob):  # selected indices are distinct; repeats become pads
        r = rows[t]
        dup = np.concatenate([[False], r[1:] == r[:-1]])
        r[dup] = -1
    got = bench.sparse_set_sizes(rows, w)
    want = np.array([len(oa.sparse_keyset(int(pos[t]), rows[t], w.window)) for t in range(w.T_glob)])
    assert np.array_equal(got, want)


def test_sparse_set_sizes_without_window():
    w = synth.custom(78, [40], [40], P=2, H=16, Dl=512, Dr=64, topk=8, window=0)
    rows = np.tile(np.array([0, 3, 5, 39, -1, -1, -1, -1], np.int32), (40, 1))
    got = bench.sparse_set_sizes(rows, w)
    want = np.array([len(oa.sparse_keyset(t, rows[t], 0)) for t in range(40)])
    assert np.array_equal(got, want) and got[0] == 1 and got[39] == 4


def test_merge_bytes_closed_form():
    """Every contributor row read once (O in bf16 and its LSE), every output row written once,
    plus the int32 map."""
    w = synth.workload(2)
    plan = hp.oracle_plan(w)
    T, P = plan.merge_src.shape
    n = int((plan.merge_src >= 0).sum())
    assert n == T  # DualChunkSwap: each token has exactly one owner rank
    row = 2 * w.Dl + 4
    assert bench.merge_bytes(plan.merge_src, w.H, w.Dl) == n * w.H * row + T * w.H * row + T * P * 4
    assert bench.merge_bytes(plan.merge_src, w.H, w.Dl, kv_splits=3) == 3 * n * w.H * row + T * w.H * row + T * P * 4


def test_measured_traffic_only_for_the_profiled_workload():
    assert bench.measured_traffic(2) == (None, None)
    att, mer = bench.measured_traffic(3)
    for v in (att, mer):
        assert v is None or v > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
