"""Top-k selection of index scores, from its definition (oracle; test infrastructure only).

A sparse query at position p attends the keys an indexer selects from its causal prefix
[0, p] ("DeepSeek-V4.1: Prefill support CP with multistream forward prepare (4/N)",
"Modifications": indexer work ahead of the MQA logits; its commit list: the indexer's
top-k). The pages do not spell the rule out; the reading taken here: the k prefix keys with
the largest scores, equal scores ordered by the smaller key index (-0 equals +0), returned as
increasing indices; a prefix of at most k keys is taken whole and padded with -1.
"""
import numpy as np


def topk_select(scores_row: np.ndarray, n: int, k: int) -> np.ndarray:
    """int64 [k]: the selected key indices of one row with n prefix keys, increasing, -1 padded."""
    if n <= k:
        return np.concatenate([np.arange(n, dtype=np.int64), np.full(k - n, -1, dtype=np.int64)])
    s = np.asarray(scores_row[:n], dtype=np.float64)
    order = np.lexsort((np.arange(n), -s))  # by score descending, then index ascending
    return np.sort(order[:k]).astype(np.int64)
