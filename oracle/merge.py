"""Log-sum-exp merge of per-rank partial attention with the sink applied once (oracle;
test infrastructure only).

Source: "[DeepSeekV4][PCP] Enable context-parallel prefill for hybrid KV and
MegaMoE", "Purpose" (each PCP rank computes a local partial attention, then LSE and
output are merged globally and attn_sink is applied only once) and "Main challenges"
(attn_sink must not be applied independently on each rank). The merged rows are put
back in global scheduled-token order ("[Core] Add MRV2 virtual-batch PCP for MLA",
"DualChunkSwap partitioning", last paragraph).

For one output row (token t, head h) with contributors k (partial output O_k over a
disjoint part of the key set, natural-log LSE L_k of that part, no sink inside) and
sink logit sigma_h:

    M   = max(sigma_h, max_k L_k)
    D   = exp(sigma_h - M) + sum_k exp(L_k - M)
    O   = sum_k exp(L_k - M) O_k / D
    LSE = M + log D

which equals attention over the union of the parts with the sink in the denominator
once, because sum_k exp(L_k) O_k = sum_j exp(S_j) v_j.
"""
import numpy as np


def merge_row(o_parts, lse_parts, sink: float):
    """o_parts: list of [Dv] arrays, lse_parts: list of floats (one entry per contributor).

    sink = -inf means no sink. An empty contributor list returns (0, sink).
    """
    L = np.asarray(lse_parts, dtype=np.float64)
    if len(L) == 0:
        return None, float(sink)
    M = max(float(sink), float(L.max()))
    w = np.exp(L - M)
    D = np.exp(float(sink) - M) + w.sum()
    O = sum(w[k] * np.asarray(o_parts[k], dtype=np.float64) for k in range(len(L))) / D
    return O, M + np.log(D)


def merge(o_cat: np.ndarray, lse_cat: np.ndarray, merge_src: np.ndarray, sink: np.ndarray):
    """Merge rank-concatenated partials into global order.

    o_cat [R, H, Dv] and lse_cat [R, H] (fp64 values of the stored partials),
    merge_src [T, P] row of o_cat contributed by each rank (-1 = none), sink [H].
    Returns O [T, H, Dv], LSE [T, H]. A row with no contributor gets O = 0, LSE = sigma.
    """
    T, P = merge_src.shape
    H, Dv = o_cat.shape[1], o_cat.shape[2]
    O = np.zeros((T, H, Dv))
    LSE = np.zeros((T, H))
    for t in range(T):
        rows = [int(x) for x in merge_src[t] if x >= 0]
        for h in range(H):
            o, l = merge_row([o_cat[r, h] for r in rows], [lse_cat[r, h] for r in rows],
                             float(sink[h]))
            if o is not None:
                O[t, h] = o
            LSE[t, h] = l
    return O, LSE
