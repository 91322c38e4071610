"""Seeded synthetic inputs for the PCP MLA prefill path.

This module only *draws* inputs: request lengths, query rows, latent/rope KV rows,
per-head sink logits and sparse key indices. It holds none of the method's
arithmetic (no partition, no attention, no merge), so both the HIP path and the
fp64 oracle consume its bytes without sharing any computation.

Every tensor is generated in row blocks, each from its own
``numpy.random.Generator(PCG64(SeedSequence([workload_seed, tensor_id, block])))``,
so any row can be regenerated on the host without materialising the whole tensor.
Floating values are drawn in fp32 and encoded to bf16 with round-to-nearest-even.

Workloads (the five shapes the path is measured and checked on):

1. tiny dense: 1 request of 256 tokens, 2 ranks, 4 heads, latent 64 + rope 16.
2. dense 8K: 1 request of 8192 tokens, 2 ranks, 16 heads, latent 512 + rope 64.
3. dense 128K: 1 request of 131072 tokens, 4 ranks, 16 heads, latent 512 + rope 64.
4. sparse 128K: 1 request of 131072 tokens, 2 ranks, 64 heads, top-2048 keys drawn
   uniformly without replacement from the causal prefix plus a 128-token window,
   latent KV stored as fp8-e4m3 with one power-of-two fp32 scale per 64 packed KV rows
   (the library's quantise-on-insert rule).
5. mixed varlen: 8 prefills with lengths log-uniform in [4096, 65536) and 64 decode
   rows (1 token each) with contexts log-uniform in [1024, 32768), 4 ranks, 16 heads.
6. chunked prefill: one step of 32768 batched tokens, 4 ranks, 16 heads: the last 16384-
   token chunk of a 131072-token prompt, an 8192-token chunk at context 40960, a fresh
   8108-token prefill, prefills at the replication threshold (8 new tokens = 2P, split;
   7 new tokens, and 5 new tokens after 895 cached ones, replicated) and 64 decode rows
   with contexts log-uniform in [1024, 32768).

q / latent / rope values ~ N(0,1)*0.5 (the fp8 latent of workload 4 ~ N(0,1)),
sink ~ N(0,1) per head, softmax scale fp32(1/sqrt(latent+rope)).

Index scores (the top-k selection's input) are not drawn from a stream but hashed from
(workload, global token, key position) with MurmurHash3's 32-bit finaliser, so any row can be
rebuilt alone, on the host (numpy) or on the device (torch integer ops, bit-identical):
score = (h >> 8) * 2^-24, uniform on a 2^-24 grid in [0, 1) (ties happen, as with real logits).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROW_BLOCK = 256  # tokens (or KV rows) per independently seeded block

# tensor ids in the seed sequence
T_Q, T_LATENT, T_ROPE, T_SINK, T_TOPK, T_LENGTHS = 0, 1, 2, 3, 4, 5

FP8_TILE = 64  # packed KV rows per fp32 scale
FP8_MAX = 448.0  # largest finite OCP E4M3FN magnitude


@dataclass
class Workload:
    cfg: int
    name: str
    q_lens: np.ndarray  # int32 [n_req]: new tokens per request (batch order)
    kv_lens: np.ndarray  # int32 [n_req]: KV rows per request, new tokens included
    P: int  # PCP size (virtual ranks)
    H: int  # query heads
    Dl: int  # latent dim (= value dim)
    Dr: int  # rope dim
    topk: int = 0  # 0 = dense causal
    window: int = 0  # sliding window added to the sparse key set (0 = none)
    kv_dtype: str = "bf16"  # "bf16" or "fp8"
    latent_std: float = 0.5
    kv_start: np.ndarray = field(default=None)  # int64 [n_req], packed KV offsets

    def __post_init__(self):
        self.q_lens = np.asarray(self.q_lens, dtype=np.int32)
        self.kv_lens = np.asarray(self.kv_lens, dtype=np.int32)
        if self.kv_start is None:
            ks = np.zeros(len(self.kv_lens), dtype=np.int64)
            ks[1:] = np.cumsum(self.kv_lens.astype(np.int64))[:-1]
            self.kv_start = ks

    @property
    def n_req(self) -> int:
        return int(len(self.q_lens))

    @property
    def Dqk(self) -> int:
        return self.Dl + self.Dr

    @property
    def T_glob(self) -> int:
        return int(self.q_lens.sum())

    @property
    def N_kv(self) -> int:
        return int(self.kv_lens.astype(np.int64).sum())

    @property
    def scale(self) -> np.float32:
        return np.float32(1.0 / math.sqrt(self.Dqk))

    @property
    def cu_q(self) -> np.ndarray:
        cu = np.zeros(self.n_req + 1, dtype=np.int64)
        cu[1:] = np.cumsum(self.q_lens.astype(np.int64))
        return cu

    def token_request(self, t: np.ndarray) -> np.ndarray:
        """Request index of global packed token(s) t (batch order, tokens by position)."""
        return np.searchsorted(self.cu_q, np.asarray(t), side="right") - 1

    def token_position(self, t: np.ndarray) -> np.ndarray:
        """Position of global token t inside its request's KV (new tokens come last)."""
        t = np.asarray(t)
        b = self.token_request(t)
        return (self.kv_lens[b] - self.q_lens[b] + (t - self.cu_q[b])).astype(np.int64)


def _config5_lengths() -> tuple[np.ndarray, np.ndarray]:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5, T_LENGTHS, 0])))
    pre = np.floor(np.exp(rng.uniform(math.log(4096), math.log(65536), 8))).astype(np.int64)
    ctx = np.floor(np.exp(rng.uniform(math.log(1024), math.log(32768), 64))).astype(np.int64)
    q = np.concatenate([pre, np.ones(64, dtype=np.int64)])
    kv = np.concatenate([pre, ctx])
    return q.astype(np.int32), kv.astype(np.int32)


def _config6_lengths() -> tuple[np.ndarray, np.ndarray]:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([6, T_LENGTHS, 0])))
    ctx = np.floor(np.exp(rng.uniform(math.log(1024), math.log(32768), 64))).astype(np.int64)
    q = np.array([16384, 8192, 8108, 8, 7, 5] + [1] * 64, dtype=np.int64)
    kv = np.concatenate([[131072, 49152, 8108, 4000, 7, 900], ctx])
    return q.astype(np.int32), kv.astype(np.int32)


def _config7_lengths() -> tuple[np.ndarray, np.ndarray]:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([7, T_LENGTHS, 0])))
    ctx = np.floor(np.exp(rng.uniform(math.log(32768), math.log(131072), 64))).astype(np.int64)
    q = np.array([4096] + [1] * 64, dtype=np.int64)
    kv = np.concatenate([[4096], ctx])
    return q.astype(np.int32), kv.astype(np.int32)


def workload(cfg: int) -> Workload:
    if cfg == 1:
        return Workload(1, "tiny dense T=256 P=2 H=4 64+16", [256], [256], P=2, H=4, Dl=64, Dr=16)
    if cfg == 2:
        return Workload(2, "dense T=8192 P=2 H=16 512+64", [8192], [8192], P=2, H=16, Dl=512, Dr=64)
    if cfg == 3:
        return Workload(3, "dense T=131072 P=4 H=16 512+64", [131072], [131072], P=4, H=16, Dl=512, Dr=64)
    if cfg == 4:
        return Workload(4, "sparse top2048+win128 fp8 T=131072 P=2 H=64 512+64", [131072], [131072],
                        P=2, H=64, Dl=512, Dr=64, topk=2048, window=128, kv_dtype="fp8", latent_std=1.0)
    if cfg == 5:
        q, kv = _config5_lengths()
        return Workload(5, "mixed varlen 8 prefill + 64 decode P=4 H=16 512+64", q, kv, P=4, H=16, Dl=512, Dr=64)
    if cfg == 6:
        q, kv = _config6_lengths()
        return Workload(6, "chunked prefill step 32768 tokens (continuations + decode) P=4 H=16 512+64", q, kv,
                        P=4, H=16, Dl=512, Dr=64)
    if cfg == 7:
        q, kv = _config7_lengths()
        return Workload(7, "decode-heavy: 64 decode rows over 32K-128K contexts + 4096-token prefill P=4 H=16 512+64",
                        q, kv, P=4, H=16, Dl=512, Dr=64)
    raise ValueError(f"unknown workload {cfg}")


def custom(cfg_seed: int, q_lens, kv_lens, P: int, H: int, Dl: int, Dr: int, **kw) -> Workload:
    """A workload of arbitrary shape (edge cases); cfg_seed keys its random streams."""
    return Workload(cfg_seed, f"custom{cfg_seed}", q_lens, kv_lens, P=P, H=H, Dl=Dl, Dr=Dr, **kw)


# --------------------------------------------------------------------------- encoding

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def _gen(cfg: int, tensor: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, tensor, block])))


def _pool_map(fn, items):
    items = list(items)
    n = min(16, os.cpu_count() or 1, max(1, len(items)))
    if n <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))


def _normal_rows(cfg: int, tensor: int, n_rows: int, row_elems: int, r0: int, r1: int,
                 std: float) -> np.ndarray:
    """fp32 rows [r0, r1) of an n_rows x row_elems N(0, std^2) tensor, block-seeded."""
    r0, r1 = max(0, r0), min(n_rows, r1)
    out = np.empty((max(0, r1 - r0), row_elems), dtype=np.float32)
    if r1 <= r0:
        return out
    blocks = range(r0 // ROW_BLOCK, (r1 - 1) // ROW_BLOCK + 1)

    def one(b):
        b0 = b * ROW_BLOCK
        nb = min(ROW_BLOCK, n_rows - b0)
        x = _gen(cfg, tensor, b).standard_normal(nb * row_elems, dtype=np.float32)
        x = x.reshape(nb, row_elems)
        if std != 1.0:
            x *= np.float32(std)
        lo, hi = max(r0, b0), min(r1, b0 + nb)
        out[lo - r0:hi - r0] = x[lo - b0:hi - b0]

    _pool_map(one, blocks)
    return out


# --------------------------------------------------------------------------- tensors

def q_rows(w: Workload, t0: int = 0, t1: int | None = None) -> np.ndarray:
    """bf16 bits [t1-t0, H, Dl+Dr] of the query rows of global tokens [t0, t1)."""
    t1 = w.T_glob if t1 is None else t1
    x = _normal_rows(w.cfg, T_Q, w.T_glob, w.H * w.Dqk, t0, t1, 0.5)
    return bf16_bits(x).reshape(-1, w.H, w.Dqk)


def rope_rows(w: Workload, r0: int = 0, r1: int | None = None) -> np.ndarray:
    """bf16 bits [r1-r0, Dr] of packed KV rows [r0, r1) (rope part of the key)."""
    r1 = w.N_kv if r1 is None else r1
    return bf16_bits(_normal_rows(w.cfg, T_ROPE, w.N_kv, w.Dr, r0, r1, 0.5))


def latent_rows(w: Workload, r0: int = 0, r1: int | None = None) -> np.ndarray:
    """Latent rows [r0, r1) of the packed KV.

    bf16 workloads: bf16 bits uint16 [n, Dl]. fp8 workloads: E4M3FN codes uint8 [n, Dl];
    their tile scales come from :func:`kv_scales`.
    """
    r1 = w.N_kv if r1 is None else r1
    if w.kv_dtype == "bf16":
        return bf16_bits(_normal_rows(w.cfg, T_LATENT, w.N_kv, w.Dl, r0, r1, w.latent_std))
    codes, _ = _fp8_tiles(w, r0 // FP8_TILE, (r1 + FP8_TILE - 1) // FP8_TILE)
    base = (r0 // FP8_TILE) * FP8_TILE
    return codes[r0 - base:r1 - base]


def kv_scales(w: Workload) -> np.ndarray:
    """fp32 scale per 64 packed KV rows (fp8 workloads only)."""
    n_tiles = (w.N_kv + FP8_TILE - 1) // FP8_TILE
    _, s = _fp8_tiles(w, 0, n_tiles, want_codes=False)
    return s


def _fp8_tiles(w: Workload, tile0: int, tile1: int, want_codes: bool = True):
    """Quantise latent tiles [tile0, tile1) to E4M3FN: scale = the smallest power of two
    (at least 2^-126) not below fp32(amax(tile)/448), 1 for an all-zero tile; RNE + saturate.

    The encoding is done by torch's float8_e4m3fn cast (a library routine): it only
    prepares the stored cache bytes, the way a cache writer would.
    """
    import torch

    r0, r1 = tile0 * FP8_TILE, min(w.N_kv, tile1 * FP8_TILE)
    x = _normal_rows(w.cfg, T_LATENT, w.N_kv, w.Dl, r0, r1, w.latent_std)
    n = r1 - r0
    nt = tile1 - tile0
    pad = nt * FP8_TILE - n
    xp = np.concatenate([x, np.zeros((pad, w.Dl), np.float32)]) if pad else x
    tiles = xp.reshape(nt, FP8_TILE * w.Dl)
    amax = np.abs(tiles).max(axis=1)
    r = (amax / np.float32(FP8_MAX)).astype(np.float32)
    m, e = np.frexp(r)  # r = m 2^e, 0.5 <= m < 1 (exact)
    scale = np.ldexp(np.float32(1.0), np.where(m == 0.5, e - 1, e)).astype(np.float32)
    scale = np.maximum(scale, np.float32(2.0**-126))
    scale[amax == 0] = np.float32(1.0)
    if not want_codes:
        return None, scale
    t = torch.from_numpy(tiles) / torch.from_numpy(scale)[:, None]
    t = torch.clamp(t, -FP8_MAX, FP8_MAX)
    codes = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(nt * FP8_TILE, w.Dl)
    return codes[:n], scale


# --------------------------------------------------------------------------- index scores

_M32 = 0xFFFFFFFF


def _fmix32(x):
    """MurmurHash3's 32-bit finaliser on uint32 numpy values (or int64 torch tensors holding
    32-bit values); wraps modulo 2^32."""
    x = x ^ (x >> 16)
    x = (x * 0x85EBCA6B) & _M32
    x = x ^ (x >> 13)
    x = (x * 0xC2B2AE35) & _M32
    return x ^ (x >> 16)


def _score_keys(cfg: int):
    return _fmix32(np.uint64((cfg * 0x9E3779B9 + 0x632BE5AB) & _M32))


def index_scores(w: Workload, tokens, n_cols: int) -> np.ndarray:
    """fp32 [len(tokens), n_cols]: index scores of the given global tokens against key
    positions 0..n_cols-1 (hash of workload, token, position; see the module header)."""
    tok = np.asarray(tokens, dtype=np.uint64)
    rk = _fmix32((tok ^ _score_keys(w.cfg)) & np.uint64(_M32))
    ck = _fmix32((np.arange(n_cols, dtype=np.uint64) * np.uint64(0x27D4EB2F)) & np.uint64(_M32))
    h = _fmix32(rk[:, None] ^ ck[None, :])
    return ((h >> np.uint64(8)).astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)


def index_scores_device(w: Workload, tokens, n_cols: int, out=None, rows_per_chunk: int = 256):
    """The same scores as :func:`index_scores`, built on the tokens' device with torch integer
    ops (chunks of rows); ``tokens`` is an int tensor, ``out`` an fp32 [len(tokens), >= n_cols]
    tensor (allocated when None)."""
    import torch

    dev = tokens.device
    T = int(tokens.shape[0])
    if out is None:
        out = torch.empty(T, n_cols, dtype=torch.float32, device=dev)
    ck = _fmix32((torch.arange(n_cols, dtype=torch.int64, device=dev) * 0x27D4EB2F) & _M32)
    key = int(_score_keys(w.cfg))
    for a in range(0, T, rows_per_chunk):
        rk = _fmix32((tokens[a:a + rows_per_chunk].to(torch.int64) ^ key) & _M32)
        h = _fmix32(rk[:, None] ^ ck[None, :])
        out[a:a + rows_per_chunk, :n_cols] = (h >> 8).to(torch.float32) * (2.0 ** -24)
    return out


def sink(w: Workload) -> np.ndarray:
    """Per-head sink logits, fp32 [H], ~ N(0,1)."""
    return _gen(w.cfg, T_SINK, 0).standard_normal(w.H, dtype=np.float32)


def _first_distinct(draws: np.ndarray, m: np.ndarray):
    """Rows of the first m[i] distinct values in each row's draw order, sorted ascending.

    Taking the first m distinct values of an i.i.d. uniform sequence gives a uniformly
    random m-subset. Returns (values sorted per row, mask of chosen) or None for rows
    with fewer than m distinct draws.
    """
    B, M = draws.shape
    order = np.argsort(draws, axis=1, kind="stable")
    sv = np.take_along_axis(draws, order, axis=1)
    first = np.ones_like(sv, dtype=bool)
    first[:, 1:] = sv[:, 1:] != sv[:, :-1]
    fidx = np.where(first, order, M)
    sf = np.sort(fidx, axis=1)
    thresh = sf[np.arange(B), m - 1]
    ok = thresh < M
    chosen = first & (order <= thresh[:, None])
    return sv, chosen, ok


def topk_rows(w: Workload, t0: int = 0, t1: int | None = None) -> np.ndarray:
    """int32 [t1-t0, topk] request-relative key positions per query token; -1 = pad.

    Each query at position p gets topk distinct positions drawn uniformly without
    replacement from [0, p] (all of [0, p] when p+1 <= topk), sorted ascending.
    """
    t1 = w.T_glob if t1 is None else t1
    k = w.topk
    out = np.full((max(0, t1 - t0), k), -1, dtype=np.int32)
    if t1 <= t0:
        return out
    blocks = range(t0 // ROW_BLOCK, (t1 - 1) // ROW_BLOCK + 1)

    def one(b):
        b0 = b * ROW_BLOCK
        nb = min(ROW_BLOCK, w.T_glob - b0)
        toks = np.arange(b0, b0 + nb)
        n = w.token_position(toks) + 1  # prefix size per query
        rng = _gen(w.cfg, T_TOPK, b)
        res = np.full((nb, k), -1, dtype=np.int32)
        small = n <= k
        for i in np.nonzero(small)[0]:
            res[i, :n[i]] = np.arange(n[i], dtype=np.int32)
        big = np.nonzero(~small)[0]
        # choose directly when n >= 2k, else choose the n-k excluded positions
        direct = big[n[big] >= 2 * k]
        compl = big[n[big] < 2 * k]
        for rows, take_complement in ((direct, False), (compl, True)):
            todo = rows
            mult = 1.5
            while len(todo):
                nn = n[todo]
                m = (nn - k) if take_complement else np.full(len(todo), k)
                M = int(math.ceil(mult * (m.max() if len(m) else 1))) + 64
                draws = rng.integers(0, nn[:, None], size=(len(todo), M), dtype=np.int64)
                sv, chosen, ok = _first_distinct(draws, m)
                for j in np.nonzero(ok)[0]:
                    i = todo[j]
                    sel = sv[j][chosen[j]]
                    if take_complement:
                        keep = np.ones(nn[j], dtype=bool)
                        keep[sel] = False
                        sel = np.nonzero(keep)[0]
                    res[i] = sel.astype(np.int32)
                todo = todo[~ok]
                mult *= 2
        lo, hi = max(t0, b0), min(t1, b0 + nb)
        out[lo - t0:hi - t0] = res[lo - b0:hi - b0]

    _pool_map(one, blocks)
    return out
