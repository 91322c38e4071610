"""Pins of the oracle's attention (dense, sparse, sink) and number decoding."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import numerics as on


def _rand(rng, *shape, s=0.5):
    return rng.standard_normal(shape) * s


def _brute(q, lat, rope, scale, sink=None):
    """Full T x T score matrix with explicit per-element loops (a different code shape)."""
    T, H, _ = q.shape
    Dl = lat.shape[1]
    O = np.zeros((T, H, Dl))
    L = np.zeros((T, H))
    for t in range(T):
        for h in range(H):
            scores = []
            for j in range(T):
                if j <= t:
                    acc = 0.0
                    for d in range(Dl):
                        acc += q[t, h, d] * lat[j, d]
                    for d in range(rope.shape[1]):
                        acc += q[t, h, Dl + d] * rope[j, d]
                    scores.append(scale * acc)
                else:
                    scores.append(None)
            den = sum(math.exp(s) for s in scores if s is not None)
            if sink is not None:
                den += math.exp(sink[h])
            num = np.zeros(Dl)
            for j, s in enumerate(scores):
                if s is not None:
                    num += math.exp(s) * lat[j]
            O[t, h] = num / den
            L[t, h] = math.log(den)
    return O, L


@pytest.mark.parametrize("T,H,Dl,Dr", [(1, 1, 4, 2), (9, 2, 8, 4), (17, 3, 6, 2)])
def test_dense_vs_brute_force(T, H, Dl, Dr):
    rng = np.random.default_rng(T * 100 + H)
    q, lat, rope = _rand(rng, T, H, Dl + Dr), _rand(rng, T, Dl), _rand(rng, T, Dr)
    sink = rng.standard_normal(H)
    scale = 1 / math.sqrt(Dl + Dr)
    o0, l0, o, l = oa.dense_causal_block(q, np.arange(T), lat, rope, scale, sink)
    bo0, bl0 = _brute(q, lat, rope, scale)
    bo, bl = _brute(q, lat, rope, scale, sink)
    np.testing.assert_allclose(o0, bo0, atol=1e-12)
    np.testing.assert_allclose(l0, bl0, atol=1e-12)
    np.testing.assert_allclose(o, bo, atol=1e-12)
    np.testing.assert_allclose(l, bl, atol=1e-12)
    # the explicit-key-set entry point agrees on every row
    for t in range(T):
        ko0, kl0, ko, kl = oa.attend_keyset(q[t], lat[:t + 1], rope[:t + 1], scale, sink)
        np.testing.assert_allclose(ko, bo[t], atol=1e-12)
        np.testing.assert_allclose(kl0, bl0[t], atol=1e-12)


def test_dense_vs_torch_sdpa():
    """Library special case: SDPA (fp64, CPU, causal) with the one KV head broadcast
    over the query heads and value dim != query dim."""
    rng = np.random.default_rng(7)
    T, H, Dl, Dr = 48, 4, 32, 8
    q, lat, rope = _rand(rng, T, H, Dl + Dr), _rand(rng, T, Dl), _rand(rng, T, Dr)
    scale = 1 / math.sqrt(Dl + Dr)
    o0, l0, _, _ = oa.dense_causal_block(q, np.arange(T), lat, rope, scale)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]  # [1, H, T, E]
    k = torch.from_numpy(np.concatenate([lat, rope], 1))[None, None].expand(1, H, T, Dl + Dr)
    v = torch.from_numpy(lat)[None, None].expand(1, H, T, Dl)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=scale)
    np.testing.assert_allclose(o0, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)
    # LSE from the library's logsumexp over the masked score matrix
    s = torch.einsum("hte,hse->hts", qt[0], k[0]) * scale
    s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(l0, torch.logsumexp(s, -1).permute(1, 0).numpy(), atol=1e-12)


def test_zero_query_closed_form():
    """q = 0: uniform weights, O_t = mean(latent_0..t), LSE = ln(t+1)."""
    rng = np.random.default_rng(3)
    T, H, Dl, Dr = 20, 2, 8, 4
    q = np.zeros((T, H, Dl + Dr))
    lat, rope = _rand(rng, T, Dl), _rand(rng, T, Dr)
    o0, l0, _, _ = oa.dense_causal_block(q, np.arange(T), lat, rope, 0.3)
    for t in range(T):
        np.testing.assert_allclose(o0[t], np.broadcast_to(lat[:t + 1].mean(0), (H, Dl)), atol=1e-13)
        np.testing.assert_allclose(l0[t], math.log(t + 1), atol=1e-13)


def test_first_row_and_identical_keys():
    rng = np.random.default_rng(4)
    T, H, Dl, Dr = 12, 3, 8, 4
    q, lat, rope = _rand(rng, T, H, Dl + Dr), _rand(rng, T, Dl), _rand(rng, T, Dr)
    s = 0.25
    o0, l0, _, _ = oa.dense_causal_block(q, np.arange(T), lat, rope, s)
    key0 = np.concatenate([lat[0], rope[0]])
    np.testing.assert_allclose(o0[0], np.broadcast_to(lat[0], (H, Dl)), atol=1e-14)
    np.testing.assert_allclose(l0[0], s * q[0] @ key0, atol=1e-13)
    # identical keys: O = latent, LSE = S + ln(n)
    lat_same = np.broadcast_to(lat[0], (T, Dl)).copy()
    rope_same = np.broadcast_to(rope[0], (T, Dr)).copy()
    o0, l0, _, _ = oa.dense_causal_block(q, np.arange(T), lat_same, rope_same, s)
    for t in range(T):
        np.testing.assert_allclose(o0[t], np.broadcast_to(lat[0], (H, Dl)), atol=1e-13)
        np.testing.assert_allclose(l0[t], s * q[t] @ key0 + math.log(t + 1), atol=1e-12)


def test_sink_closed_form():
    """O = O0 * logistic(LSE0 - sigma), LSE = logaddexp(LSE0, sigma); sigma=-inf -> no sink."""
    rng = np.random.default_rng(5)
    T, H, Dl, Dr = 16, 4, 8, 4
    q, lat, rope = _rand(rng, T, H, Dl + Dr), _rand(rng, T, Dl), _rand(rng, T, Dr)
    sink = np.array([-1.0, 0.0, 2.5, 6.0])
    o0, l0, o, l = oa.dense_causal_block(q, np.arange(T), lat, rope, 0.3, sink)
    w = 1.0 / (1.0 + np.exp(-(l0 - sink[None, :])))
    np.testing.assert_allclose(o, o0 * w[..., None], atol=1e-13)
    np.testing.assert_allclose(l, np.logaddexp(l0, sink[None, :]), atol=1e-13)
    _, _, o_inf, l_inf = oa.dense_causal_block(q, np.arange(T), lat, rope, 0.3,
                                               np.full(H, -np.inf))
    np.testing.assert_allclose(o_inf, o0, atol=1e-15)
    np.testing.assert_allclose(l_inf, l0, atol=1e-15)


def test_sparse_reduces_to_dense_and_window():
    rng = np.random.default_rng(6)
    T, H, Dl, Dr, W = 40, 2, 8, 4, 5
    q, lat, rope = _rand(rng, T, H, Dl + Dr), _rand(rng, T, Dl), _rand(rng, T, Dr)
    o0, l0, _, _ = oa.dense_causal_block(q, np.arange(T), lat, rope, 0.3)
    for p in range(T):
        # selected indices covering the whole prefix (shuffled, padded) -> dense
        sel = np.concatenate([rng.permutation(p + 1), -np.ones(3, int)])
        ks = oa.sparse_keyset(p, sel, W)
        assert np.array_equal(ks, np.arange(p + 1))
        ko0, kl0, _, _ = oa.attend_keyset(q[p], lat[ks], rope[ks], 0.3)
        np.testing.assert_allclose(ko0, o0[p], atol=1e-13)
        np.testing.assert_allclose(kl0, l0[p], atol=1e-13)
        # nothing selected -> sliding window only, checked against a banded-mask brute force
        ks = oa.sparse_keyset(p, -np.ones(4, int), W)
        assert np.array_equal(ks, np.arange(max(0, p - W + 1), p + 1))
        lo = max(0, p - W + 1)
        so = 0.3 * (q[p, :, :Dl] @ lat.T + q[p, :, Dl:] @ rope.T)
        band = (np.arange(T) >= lo) & (np.arange(T) <= p)
        so[:, ~band] = -np.inf
        e = np.exp(so - so.max(1, keepdims=True))
        want = (e @ lat) / e.sum(1, keepdims=True)
        ko0, _, _, _ = oa.attend_keyset(q[p], lat[ks], rope[ks], 0.3)
        np.testing.assert_allclose(ko0, want, atol=1e-13)


def test_sparse_union_counts_once():
    p, W = 100, 8
    sel = np.array([3, 50, 95, 97, 100, -1, -1])  # 95, 97, 100 fall inside the window
    ks = oa.sparse_keyset(p, sel, W)
    assert list(ks) == [3, 50] + list(range(93, 101))
    assert len(ks) == len(set(sel[sel >= 0]) | set(range(93, 101)))


def test_e4m3fn_table_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = on.e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.nanmax(mine) == 448.0 and mine[0x01] == 2.0 ** -9
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0,
                                  1e-40, 3.0e38], np.float32)])
    bits = x.view(np.uint32)
    # force exact ties in a slice
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000
    x = bits.view(np.float32)
    mine = on.f32_to_bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x4049, 0x0001], np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(on.bf16_to_f64(bits), want)


def test_fp8_dequant_rounding():
    codes = np.arange(256, dtype=np.uint8).reshape(4, 64)
    scales = np.array([0.37, 1.0 / 448], np.float32)
    rows = np.array([0, 63, 64, 127])
    got = on.dequant_fp8_rows(codes, rows, scales)
    dec = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32)
    s = torch.from_numpy(scales)[torch.from_numpy(rows) // 64]
    ref = (dec * s[:, None]).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def _loop_attend(q_tok, lat_keys, rope_keys, scale, sink):
    """Per-head explicit loops over an explicit key list (no matrix products)."""
    H = q_tok.shape[0]
    Dl = lat_keys.shape[1]
    O = np.zeros((H, Dl))
    L = np.zeros(H)
    for h in range(H):
        sc = [scale * (float(q_tok[h, :Dl] @ lat_keys[j]) + float(q_tok[h, Dl:] @ rope_keys[j]))
              for j in range(len(lat_keys))]
        den = sum(math.exp(x) for x in sc) + (0.0 if sink is None else math.exp(sink[h]))
        O[h] = sum(math.exp(x) * lat_keys[j] for j, x in enumerate(sc)) / den
        L[h] = math.log(den)
    return O, L


@pytest.mark.parametrize("block", [1, 3, 256])
def test_attention_tokens_multi_request_batch(block):
    """The oracle's batch driver on a packed batch of several requests: fresh prefills,
    continuations (kv_len > q_len, context already cached), a short prefill and decode rows,
    with KV segments at non-zero, gapped starts and the tokens asked in shuffled order.
    Every token must equal its own request's causal prefix, attended alone: position
    kv_len - q_len + i of request b attends packed rows kv_start[b] .. kv_start[b] + position
    ("[Core] Add MRV2 virtual-batch PCP for MLA", "PCP algorithm": each request is handled on
    its own; decode rows attend their whole context)."""
    rng = np.random.default_rng(11)
    H, Dl, Dr = 3, 8, 4
    q_lens = np.array([13, 5, 1, 2, 1, 7])
    kv_lens = np.array([13, 20, 9, 2, 1, 30])
    kv_start = np.array([4, 40, 17, 70, 0, 80])  # gapped and out of batch order
    n_kv = int((kv_start + kv_lens).max()) + 3
    lat, rope = _rand(rng, n_kv, Dl), _rand(rng, n_kv, Dr)
    T = int(q_lens.sum())
    q = _rand(rng, T, H, Dl + Dr)
    sink = np.array([0.5, -1.0, 2.0])
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    req = np.repeat(np.arange(len(q_lens)), q_lens)
    pos = np.concatenate([np.arange(k - n, k) for n, k in zip(q_lens, kv_lens)])
    tokens = rng.permutation(T)
    out = oa.attention_tokens(tokens, q_of=lambda ts: q[ts], pos_of=lambda ts: pos[ts],
                              req_of=lambda ts: req[ts], kv_start=kv_start,
                              lat_rows=lambda a, b: lat[a:b], rope_rows=lambda a, b: rope[a:b],
                              scale=0.3, sink=sink, block=block)
    assert sorted(out) == list(range(T))
    for t in range(T):
        b, p = int(req[t]), int(pos[t])
        assert cu[b] <= t < cu[b + 1]
        rows = kv_start[b] + np.arange(p + 1)
        o0, l0, o, l = out[t]
        ko0, kl0, ko, kl = oa.attend_keyset(q[t], lat[rows], rope[rows], 0.3, sink)
        np.testing.assert_allclose(o0, ko0, atol=1e-12)
        np.testing.assert_allclose(l0, kl0, atol=1e-12)
        np.testing.assert_allclose(o, ko, atol=1e-12)
        np.testing.assert_allclose(l, kl, atol=1e-12)
        # and against explicit loops over the same key rows
        bo, bl = _loop_attend(q[t], lat[rows], rope[rows], 0.3, sink)
        np.testing.assert_allclose(o, bo, atol=1e-12)
        np.testing.assert_allclose(l, bl, atol=1e-12)
        bo0, bl0 = _loop_attend(q[t], lat[rows], rope[rows], 0.3, None)
        np.testing.assert_allclose(o0, bo0, atol=1e-12)
        np.testing.assert_allclose(l0, bl0, atol=1e-12)


def test_attention_tokens_subset_and_isolation():
    """Asking for a subset gives the same rows as asking for all of them, and a request's
    rows do not change when another request's KV changes (request isolation)."""
    rng = np.random.default_rng(12)
    H, Dl, Dr = 2, 8, 4
    q_lens, kv_lens, kv_start = np.array([6, 4]), np.array([6, 9]), np.array([0, 6])
    lat, rope = _rand(rng, 15, Dl), _rand(rng, 15, Dr)
    q = _rand(rng, 10, H, Dl + Dr)
    req = np.repeat([0, 1], q_lens)
    pos = np.concatenate([np.arange(6), np.arange(5, 9)])

    def run(lat_, toks):
        return oa.attention_tokens(toks, q_of=lambda ts: q[ts], pos_of=lambda ts: pos[ts],
                                   req_of=lambda ts: req[ts], kv_start=kv_start,
                                   lat_rows=lambda a, b: lat_[a:b], rope_rows=lambda a, b: rope[a:b],
                                   scale=0.4)

    full = run(lat, np.arange(10))
    part = run(lat, np.array([9, 2, 6]))
    for t in (9, 2, 6):
        for a, b in zip(full[t], part[t]):
            np.testing.assert_array_equal(a, b)
    lat2 = lat.copy()
    lat2[6:] += 1.0  # request 1's KV only
    other = run(lat2, np.arange(6))
    for t in range(6):
        for a, b in zip(full[t], other[t]):
            np.testing.assert_array_equal(a, b)


def test_sparse_keyset_drops_indices_past_the_query():
    """Selected indices after the query's position are not in its causal prefix and act as
    pads, as do negative ones; duplicates and window members count once."""
    p, W = 10, 4
    sel = np.array([3, 8, 11, 15, -1, 3, 10, 0, -7, 10 ** 6, 9])
    assert list(oa.sparse_keyset(p, sel, W)) == [0, 3, 7, 8, 9, 10]
    # every index past p at p = 0 leaves the window alone
    assert list(oa.sparse_keyset(0, np.array([1, 2, 5]), W)) == [0]
    # no window: only the selected prefix keys, deduplicated
    assert list(oa.sparse_keyset(p, sel, 0)) == [0, 3, 8, 9, 10]
    # brute-force membership on random rows
    rng = np.random.default_rng(13)
    for _ in range(200):
        p = int(rng.integers(0, 50))
        W = int(rng.integers(0, 20))
        sel = rng.integers(-3, 70, size=int(rng.integers(0, 30)))
        want = sorted({int(x) for x in sel if 0 <= x <= p} | {j for j in range(p + 1) if j > p - W})
        assert list(oa.sparse_keyset(p, sel, W)) == want
