"""CPU model of how the sparse kernel (csrc/attn_sparse_wide.hip) walks a token's key set.

The model restates the kernel's index arithmetic: the 64-bit mask of live selected-index tiles
(entries tid + 128 j of a 128-thread workgroup, one ballot per half-wave), the contiguous range
of live window tiles, the tile order (next_tile) and which slots of a tile count (stage b).
Against the oracle's key set (restricted to a split's key range) on random rows, at sizes the
GPU tests only sample: every key of the set is visited exactly once, nothing else counts, every
visited tile holds a key, and every skipped tile holds none.
"""
import numpy as np
import pytest

from oracle import attention as oa

TK = 32          # key slots per tile
NTW = 128        # threads per workgroup
MAX_TOPK = 2048


def live_mask(row, p, window, key_lo, key_hi):
    """The kernel's mask: thread tid = 64 wave + lane holds entries tid + 128 j; a ballot over
    the wave sets bit 4 j + 2 wave from lanes 0-31 and bit 4 j + 2 wave + 1 from lanes 32-63."""
    topk = len(row)
    win_lo = max(0, p - window + 1)

    def ok(e):
        return key_lo <= e < key_hi and e <= p and (window == 0 or e < win_lo)

    live = 0
    for j in range(MAX_TOPK // NTW):
        for wave in range(2):
            lanes = [ok(row[i]) if (i := 64 * wave + lane + NTW * j) < topk else False for lane in range(64)]
            t = 4 * j + 2 * wave
            live |= (any(lanes[:32]) << t) | (any(lanes[32:]) << (t + 1))
    return live


def walk(row, p, window, key_lo, key_hi):
    """Tiles the kernel visits, in order, and the keys that count in each."""
    topk = len(row)
    win_lo = max(0, p - window + 1)
    n_sel = (topk + TK - 1) // TK
    t_end = n_sel + (window + TK - 1) // TK
    a, b = max(win_lo, key_lo), min(p + 1, key_hi)
    if window > 0 and a < b:
        w_first, w_last = n_sel + (a - win_lo) // TK, n_sel + (b - 1 - win_lo) // TK
    else:
        w_first, w_last = t_end, -1
    live = live_mask(row, p, window, key_lo, key_hi)

    def next_tile(t):
        t1 = t + 1
        if t1 < n_sel:
            m = live & ~((1 << t1) - 1)
            if m:
                return (m & -m).bit_length() - 1
        w = max(t1, w_first)
        return w if w <= w_last else t_end

    def slot_keys(t):
        out = []
        for slot in range(TK):
            if t < n_sel:
                i = t * TK + slot
                e = row[i] if i < topk else -1
                if key_lo <= e < key_hi and e <= p and (window == 0 or e < win_lo):
                    out.append(int(e))
            else:
                w = (t - n_sel) * TK + slot
                k = win_lo + w
                if t < t_end and w < window and k <= p and key_lo <= k < key_hi:
                    out.append(k)
        return out

    visited = []
    t = next_tile(-1)
    while t < t_end:
        visited.append(t)
        t = next_tile(t)
    return visited, {t: slot_keys(t) for t in range(t_end)}


def split_ranges(L, S):
    """Whole 64-key tiles [64 floor(s n / S), 64 floor((s+1) n / S)) of a row of L keys."""
    n = -(-L // 64)
    return [(64 * (s * n // S), 64 * ((s + 1) * n // S)) for s in range(S)]


def random_row(rng, p, topk, kind):
    if kind == "prefix":  # every key of a short prefix, then pads (what the selection gives)
        k = min(topk, p + 1)
        row = np.full(topk, -1, np.int64)
        row[:k] = np.sort(rng.choice(p + 1, size=k, replace=False))
        return row
    k = min(topk, p + 1)
    sel = rng.choice(p + 1, size=k, replace=False)
    row = np.concatenate([sel, np.full(topk - k, -1)])
    if kind == "junk":  # out-of-range entries the kernel must treat as pads
        bad = rng.random(topk) < 0.2
        row[bad] = rng.choice([-7, p + 1, p + 1000, 1 << 30], size=int(bad.sum()))
    return rng.permutation(row) if kind != "sorted" else np.sort(row)


@pytest.mark.parametrize("seed", range(40))
def test_walk_visits_the_key_set(seed):
    rng = np.random.default_rng(seed)
    topk = int(rng.choice([1, 5, 32, 33, 64, 100, 512, 2048]))
    window = int(rng.choice([0, 1, 31, 32, 128, 300, 4096]))
    p = int(rng.choice([0, 3, 31, 32, 200, 2047, 2048, 5000, 131071]))
    kind = str(rng.choice(["sorted", "shuffled", "junk", "prefix"]))
    row = random_row(rng, p, topk, kind)
    L = p + 1 + int(rng.integers(0, 100))
    S = int(rng.choice([1, 2, 3, 5]))
    full = oa.sparse_keyset(p, row, window)
    ranges = split_ranges(L, S) if S > 1 else [(0, 2**31 - 1)]
    seen_all = []
    for key_lo, key_hi in ranges:
        visited, keys = walk(row, p, window, key_lo, key_hi)
        got = [k for t in visited for k in keys[t]]
        want = full[(full >= key_lo) & (full < key_hi)]
        assert sorted(got) == want.tolist(), (seed, key_lo, key_hi)
        assert len(got) == len(set(got))  # once each
        assert all(keys[t] for t in visited), "a visited tile holds no key"
        skipped = set(range(len(keys))) - set(visited)
        assert not any(keys[t] for t in skipped), "a skipped tile holds a key"
        seen_all += got
    assert sorted(seen_all) == full.tolist()  # the split ranges partition the key set


def test_walk_edge_rows():
    """A row whose selected indices all fall inside the window, all pads, and the window only."""
    p, window = 1000, 4096
    row = np.arange(0, 64)
    visited, keys = walk(row, p, window, 0, 2**31 - 1)
    assert all(t >= 2 for t in visited)  # the 2 selected tiles hold no key: the window has them
    assert sorted(k for t in visited for k in keys[t]) == list(range(p + 1))
    visited, _ = walk(np.full(2048, -1), 0, 0, 0, 2**31 - 1)
    assert visited == []  # no key at all: O = 0, LSE = -inf
    visited, keys = walk(np.full(1, -1), 70, 128, 0, 2**31 - 1)
    assert visited == [1, 2, 3] and sorted(k for t in visited for k in keys[t]) == list(range(71))
