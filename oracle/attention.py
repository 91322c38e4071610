"""Single-pass MLA softmax attention with a per-head sink, in fp64 (oracle; test
infrastructure only).

Absorbed MLA is multi-query attention with one latent KV head shared by every query
head: the key of KV row j is latent_j || rope_j (Dl + Dr), its value is latent_j (Dl).
Each query head h carries an already-absorbed Dl + Dr vector. This is the reading of
"K and V, or latent KV in the case of MLA, are all-gathered" ("[Core] Add MRV2
virtual-batch PCP for MLA", "DualChunkSwap partitioning") with the dimensions of the
workloads (latent 512 + rope 64, value 512).

For a query at position p of a request and head h, with key set K (causal: all keys
of the same request at positions 0..p, diagonal included; sparse: the selected set):

    S_j   = scale * <q_h, key_j>                     for j in K
    O0    = sum_j exp(S_j) latent_j / sum_j exp(S_j)   (no sink: what one rank returns)
    LSE0  = log sum_j exp(S_j)                          (natural log)

and with the per-head sink logit sigma_h (a logit in the same scaled domain with no
value vector; sigma = -inf means no sink):

    O     = sum_j exp(S_j) latent_j / (exp(sigma_h) + sum_j exp(S_j))
    LSE   = log(exp(sigma_h) + sum_j exp(S_j))

The sink enters the final denominator once ("[DeepSeekV4][PCP] Enable context-
parallel prefill for hybrid KV and MegaMoE", "Purpose": merge LSE/output globally and
apply attn_sink only once; "Main challenges": attn_sink must not be applied on each
rank). Maxima are subtracted before exponentiation for range only; that changes no
value.
"""
import numpy as np


def _softmax_stats(s: np.ndarray, v: np.ndarray, sink):
    """s: [..., n] scores (masked entries = -inf); v: [n, Dv]. Returns O0, LSE0, O, LSE."""
    m = s.max(axis=-1)
    e = np.exp(s - m[..., None])
    l = e.sum(axis=-1)
    o0 = (e @ v) / l[..., None]
    lse0 = m + np.log(l)
    if sink is None:
        return o0, lse0, o0.copy(), lse0.copy()
    sig = np.asarray(sink, dtype=np.float64)
    sig = np.broadcast_to(sig, m.shape)
    m2 = np.maximum(m, sig)
    e2 = np.exp(s - m2[..., None])
    l2 = np.exp(sig - m2) + e2.sum(axis=-1)
    o = (e2 @ v) / l2[..., None]
    lse = m2 + np.log(l2)
    return o0, lse0, o, lse


def attend_keyset(q_tok: np.ndarray, lat_keys: np.ndarray, rope_keys: np.ndarray,
                  scale: float, sink=None):
    """One query token against an explicit key set.

    q_tok [H, Dl+Dr], lat_keys [n, Dl], rope_keys [n, Dr] (fp64). Returns
    (O0 [H, Dl], LSE0 [H], O [H, Dl], LSE [H]).
    """
    Dl = lat_keys.shape[1]
    s = scale * (q_tok[:, :Dl] @ lat_keys.T + q_tok[:, Dl:] @ rope_keys.T)
    return _softmax_stats(s, lat_keys, sink)


def dense_causal_block(q_blk: np.ndarray, pos_blk: np.ndarray, lat_req: np.ndarray,
                       rope_req: np.ndarray, scale: float, sink=None):
    """Several query tokens of ONE request against that request's causal prefix.

    q_blk [n, H, Dl+Dr]; pos_blk [n] positions; lat_req / rope_req: the request's KV rows
    from position 0 on. Keys past a query's position get score -inf (exp -> 0 exactly),
    which is the causal rule written as a mask.
    Returns (O0 [n,H,Dl], LSE0 [n,H], O [n,H,Dl], LSE [n,H]).
    """
    n_keys = int(pos_blk.max()) + 1
    lat = lat_req[:n_keys]
    rope = rope_req[:n_keys]
    Dl = lat.shape[1]
    s = scale * (np.einsum("thd,kd->thk", q_blk[:, :, :Dl], lat, optimize=True)
                 + np.einsum("thd,kd->thk", q_blk[:, :, Dl:], rope, optimize=True))
    masked = np.arange(n_keys)[None, :] > pos_blk[:, None]  # [n, keys]
    s[np.broadcast_to(masked[:, None, :], s.shape)] = -np.inf
    sink_b = None if sink is None else np.asarray(sink, dtype=np.float64)[None, :]
    return _softmax_stats(s, lat, sink_b)


def sparse_keyset(p: int, topk_row: np.ndarray, window: int) -> np.ndarray:
    """Sorted request-relative key positions of a sparse query at position p.

    The set union of the selected indices (-1 = pad; entries outside [0, p] are
    treated as pads since they are not in the causal prefix) and the sliding window
    [max(0, p-window+1), p]. A selected index inside the window counts once.
    """
    sel = np.asarray(topk_row, dtype=np.int64)
    sel = sel[(sel >= 0) & (sel <= p)]
    win = np.arange(max(0, p - window + 1), p + 1, dtype=np.int64) if window > 0 else np.zeros(0, np.int64)
    return np.union1d(sel, win)


def attention_tokens(tokens, q_of, pos_of, req_of, kv_start, lat_rows, rope_rows,
                     scale, sink=None, block=256):
    """Dense causal attention for a list of global tokens.

    q_of(ts) -> fp64 [n, H, Dqk]; pos_of(ts), req_of(ts) -> int arrays;
    lat_rows(r0, r1) / rope_rows(r0, r1) -> fp64 packed KV rows.
    Tokens are grouped by request and processed ``block`` at a time (each token's
    softmax still runs over its whole key set in one pass).
    Returns dict token -> (O0, LSE0, O, LSE).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    out = {}
    reqs = req_of(tokens)
    for b in np.unique(reqs):
        tb = tokens[reqs == b]
        pb = pos_of(tb)
        order = np.argsort(pb)
        tb, pb = tb[order], pb[order]
        kv0 = int(kv_start[b])
        n_keys = int(pb.max()) + 1
        lat = lat_rows(kv0, kv0 + n_keys)
        rope = rope_rows(kv0, kv0 + n_keys)
        for i in range(0, len(tb), block):
            ts, ps = tb[i:i + block], pb[i:i + block]
            o0, l0, o, l = dense_causal_block(q_of(ts), ps, lat, rope, scale, sink)
            for j, t in enumerate(ts):
                out[int(t)] = (o0[j], l0[j], o[j], l[j])
    return out
