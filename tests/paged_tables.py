"""Block tables of the paged-cache tests (host-side set-up, shared by the GPU tests and the
CPU access model of their launches)."""
from __future__ import annotations

import numpy as np


def make_block_table(w, seed, spare=5, pad=2):
    """Each request's ceil(kv_len / 64) blocks drawn without replacement from a pool with
    spare blocks, in random order; pad columns hold -1 and are never read."""
    rng = np.random.default_rng(seed)
    nb = (w.kv_lens.astype(np.int64) + 63) // 64
    n_blocks = int(nb.sum()) + spare
    perm = rng.permutation(n_blocks)
    bt = np.full((w.n_req, int(nb.max(initial=0)) + pad), -1, np.int32)
    k = 0
    for b in range(w.n_req):
        bt[b, :nb[b]] = perm[k:k + nb[b]]
        k += int(nb[b])
    return bt, n_blocks


def corrupt_table(bt, n_blocks, b):
    """Request b's first three block-table entries replaced by ids outside the cache: past its
    end, negative, and 2^24 (its rows, 2^30 and up, still fit int32)."""
    bad = bt.copy()
    bad[b, :3] = [n_blocks + 5, -3, 1 << 24]
    return bad


def rank_order(plan):
    """Global tokens in rank-concatenated row order."""
    return np.concatenate([rp.local_gidx for rp in plan.ranks]).astype(np.int64)


def request_rows(plan, lo, hi):
    """Rank-concatenated rows of the global tokens [lo, hi)."""
    g = rank_order(plan)
    return np.nonzero((g >= lo) & (g < hi))[0]


# The workloads of the out-of-cache block-id test: a dense batch (bf16 cache) and a sparse
# batch whose bf16 latent rows the library quantises to fp8 on insert.
OUT_OF_CACHE_DENSE = dict(cfg_seed=404, q_lens=[600, 400], kv_lens=[600, 400], P=2, H=16, Dl=512, Dr=64)
OUT_OF_CACHE_SPARSE = dict(cfg_seed=504, q_lens=[700, 500], kv_lens=[700, 500], P=2, H=64, Dl=512, Dr=64,
                           topk=128, window=64, kv_dtype="bf16", latent_std=1.0)
