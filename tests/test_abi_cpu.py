"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, sizes
plans like the oracle, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from context_mla_prefill_amd import _lib
from oracle import partition as op

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_pcp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:mla_status|int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    names = _declared()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version():
    assert _lib.mla_pcp_abi_version() == _lib.ABI_VERSION


@pytest.mark.parametrize("seed", range(30))
@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
def test_plan_sizes_match_oracle(seed, P):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 12))
    q = rng.integers(0, 70, size=n)
    kv = q + rng.integers(0, 5, size=n)
    T_loc, nv, tg = _lib.pcp_plan_sizes(q, kv, P)
    plan = op.partition(q, kv, np.zeros(n, int), P)
    assert tg == plan.T_glob
    assert T_loc == [rp.T_loc for rp in plan.ranks]
    assert all(nv == rp.n_vrows for rp in plan.ranks)


def _status(fn):
    try:
        fn()
    except _lib.MlaError as e:
        return e.status, str(e)
    return 0, ""


def test_plan_sizes_errors():
    assert _status(lambda: _lib.pcp_plan_sizes([4], [3], 2))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _status(lambda: _lib.pcp_plan_sizes([4], [4], 0))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _status(lambda: _lib.pcp_plan_sizes([4], [4], 65))[0] == _lib.MLA_ERR_INVALID_ARG
    assert _status(lambda: _lib.pcp_plan_sizes([-1], [4], 2))[0] == _lib.MLA_ERR_INVALID_ARG
    big = np.full(3, 2 ** 30, dtype=np.int64).astype(np.int32)
    assert _status(lambda: _lib.pcp_plan_sizes(big, big, 2))[0] == _lib.MLA_ERR_INVALID_ARG


def _args(**kw):
    base = dict(q=None, latent_kv=None, rope_k=None, cu_seqlens_q=None, vrow_kv_start=None, positions=None,
                n_vrows=1, T_loc=4, H=16, D_latent=512, D_rope=64, scale=1 / 24, o_partial=None, lse=None,
                N_kv=16)
    base.update(kw)
    return _lib.make_partial_args(**base)


FAKE = 1 << 20  # a non-null, 16-byte aligned address; never dereferenced on these paths


class _P:
    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def test_partial_validation_errors():
    call = lambda a: _status(lambda: _lib.mla_prefill_partial(a, stream=0))
    assert call(_args())[0] == _lib.MLA_ERR_INVALID_ARG  # null pointers
    f = _P(FAKE)
    ok = dict(q=f, latent_kv=f, rope_k=f, cu_seqlens_q=f, vrow_kv_start=f, positions=f, o_partial=f, lse=f)
    assert call(_args(**ok, D_latent=128))[0] == _lib.MLA_ERR_UNSUPPORTED
    assert call(_args(**ok, H=0))[0] == _lib.MLA_ERR_UNSUPPORTED
    assert call(_args(**ok, H=129))[0] == _lib.MLA_ERR_UNSUPPORTED
    assert call(_args(**ok, scale=0.0))[0] == _lib.MLA_ERR_INVALID_ARG
    assert call(_args(**ok, scale=float("nan")))[0] == _lib.MLA_ERR_INVALID_ARG
    assert call(_args(**ok, T_loc=-1))[0] == _lib.MLA_ERR_INVALID_ARG
    assert call(_args(**ok, n_vrows=0))[0] == _lib.MLA_ERR_INVALID_ARG
    assert call(_args(**ok, kv_dtype=7))[0] == _lib.MLA_ERR_UNSUPPORTED
    assert call(_args(**{**ok, "q": _P(FAKE + 2)}))[0] == _lib.MLA_ERR_INVALID_ARG  # misaligned
    assert call(_args(**ok, kv_dtype=_lib.MLA_KV_FP8_E4M3))[0] == _lib.MLA_ERR_UNSUPPORTED  # dense fp8
    assert call(_args(**ok, topk_idx=f, topk=4096, kv_dtype=1, kv_scale=f, H=64))[0] == _lib.MLA_ERR_UNSUPPORTED
    assert call(_args(**ok, topk_idx=f, topk=2048, kv_dtype=1, H=64))[0] == _lib.MLA_ERR_INVALID_ARG  # no scale
    # the sparse path takes any head count up to 128 (head groups of up to 64 rows); H above
    # 128 is refused for both paths
    assert call(_args(**ok, topk_idx=f, topk=2048, kv_dtype=1, kv_scale=f, H=129))[0] == _lib.MLA_ERR_UNSUPPORTED
    assert call(_args(**ok, topk_idx=f, topk=2048, kv_dtype=0, H=64, N_kv=1 << 22))[0] == \
        _lib.MLA_ERR_UNSUPPORTED  # bf16 sparse rows addressed by 32-bit byte offsets
    assert call(_args(**ok, topk_idx=f, topk=2048, kv_dtype=0, H=64, D_latent=64, D_rope=16))[0] == \
        _lib.MLA_ERR_UNSUPPORTED  # sparse needs 512+64
    assert call(_args(**ok, topk_idx=f, topk=64, window=5000, kv_dtype=1, kv_scale=f, H=64))[0] == \
        _lib.MLA_ERR_UNSUPPORTED
    assert call(_args(**ok, topk_idx=f, topk=64, window=128, kv_dtype=1, kv_scale=f, H=64, N_kv=1 << 23))[0] == \
        _lib.MLA_ERR_UNSUPPORTED  # sparse KV rows addressed by 32-bit byte offsets
    assert call(_args(**ok, kv_splits=0))[0] == _lib.MLA_ERR_INVALID_ARG
    assert call(_args(**ok, kv_splits=65))[0] == _lib.MLA_ERR_INVALID_ARG
    assert call(_args(**ok, kv_splits=2, split_stride=4))[0] == _lib.MLA_ERR_INVALID_ARG  # no vrow_kv_len
    assert call(_args(**ok, kv_splits=2, split_stride=3, vrow_kv_len=f))[0] == _lib.MLA_ERR_INVALID_ARG  # < T_loc
    assert call(_args(**ok, block_table=f, bt_stride=4))[0] == _lib.MLA_ERR_INVALID_ARG  # no vrow_req
    assert call(_args(**ok, block_table=f, bt_stride=0, vrow_req=f))[0] == _lib.MLA_ERR_INVALID_ARG
    st, msg = call(_args(**ok, block_table=f, bt_stride=4, vrow_req=f))  # N_kv = 16: a partial block
    assert st == _lib.MLA_ERR_INVALID_ARG and "64-row blocks" in msg
    st, msg = call(_args(**{**ok, "N_kv": 0}))
    assert st == _lib.MLA_ERR_INVALID_ARG and "empty KV" in msg
    st, msg = call(_args(**ok, D_rope=32))
    assert st == _lib.MLA_ERR_UNSUPPORTED and "dims" in msg
    # empty shard: nothing to do, OK without touching any pointer
    assert call(_args(T_loc=0, n_vrows=0))[0] == 0


def test_merge_and_insert_validation_errors():
    f = _P(FAKE)
    m = lambda **kw: _status(lambda: _lib.pcp_lse_merge(**{**dict(
        o_cat=f, lse_cat=f, merge_src=f, P=2, T_glob=4, H=4, D_v=64, R_total=8, sink=None, o_out=f,
        lse_out=None, stream=0), **kw}))
    assert m(P=0)[0] == _lib.MLA_ERR_INVALID_ARG
    assert m(D_v=12)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert m(merge_src=None)[0] == _lib.MLA_ERR_INVALID_ARG
    assert m(o_out=_P(FAKE + 4))[0] == _lib.MLA_ERR_INVALID_ARG
    assert m(T_glob=0)[0] == 0
    assert m(kv_splits=0)[0] == _lib.MLA_ERR_INVALID_ARG
    assert m(P=8, kv_splits=9)[0] == _lib.MLA_ERR_INVALID_ARG  # 72 contributors per token
    assert m(kv_splits=2, split_stride=-1)[0] == _lib.MLA_ERR_INVALID_ARG
    ins = lambda **kw: _status(lambda: _lib.pcp_kv_insert(**{**dict(
        local_latent=f, local_rope=f, slot=f, T_loc=4, D_latent=512, D_rope=64, kv_dtype=0, N_kv=8,
        kv_latent=f, kv_rope=f, stream=0), **kw}))
    assert ins(D_latent=100)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert ins(kv_dtype=3)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert ins(slot=None)[0] == _lib.MLA_ERR_INVALID_ARG
    assert ins(T_loc=-2)[0] == _lib.MLA_ERR_INVALID_ARG
    assert ins(T_loc=0)[0] == 0
    q8 = lambda **kw: _status(lambda: _lib.pcp_kv_insert_fp8(**{**dict(
        local_latent=f, local_rope=f, slot=f, T=4, D_latent=512, D_rope=64, N_kv=128, kv_latent=f,
        kv_rope=f, kv_scale=f, stream=0), **kw}))
    assert q8(D_latent=128)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert q8(D_latent=64)[0] == _lib.MLA_ERR_UNSUPPORTED  # 64 latent goes with 16 rope
    assert q8(T=-1)[0] == _lib.MLA_ERR_INVALID_ARG
    assert q8(N_kv=1 << 31)[0] == _lib.MLA_ERR_INVALID_ARG
    assert q8(kv_scale=None)[0] == _lib.MLA_ERR_INVALID_ARG
    assert q8(local_latent=_P(FAKE + 8))[0] == _lib.MLA_ERR_INVALID_ARG
    assert q8(T=0)[0] == 0


def test_dequant_validation_errors():
    f = _P(FAKE)
    dq = lambda **kw: _status(lambda: _lib.pcp_kv_dequant_fp8(**{**dict(
        kv_latent=f, kv_scale=f, N_kv=128, D_latent=512, blocks=f, n_blocks=2, ws=f, stream=0), **kw}))
    assert dq(D_latent=128)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert dq(N_kv=-1)[0] == _lib.MLA_ERR_INVALID_ARG
    assert dq(n_blocks=-1)[0] == _lib.MLA_ERR_INVALID_ARG
    assert dq(blocks=None)[0] == _lib.MLA_ERR_INVALID_ARG
    assert dq(ws=_P(FAKE + 2))[0] == _lib.MLA_ERR_INVALID_ARG
    assert dq(n_blocks=0)[0] == 0 and dq(N_kv=0)[0] == 0


def test_topk_select_validation_errors():
    f = _P(FAKE)
    sel = lambda **kw: _status(lambda: _lib.sparse_topk_select(**{**dict(
        scores=f, ld=4096, positions=f, T=8, k=2048, topk_idx=f, stream=0), **kw}))
    assert sel(k=0)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert sel(k=2049)[0] == _lib.MLA_ERR_UNSUPPORTED
    assert sel(ld=4094)[0] == _lib.MLA_ERR_INVALID_ARG  # rows not 16-byte aligned
    assert sel(ld=0)[0] == _lib.MLA_ERR_INVALID_ARG
    assert sel(T=-1)[0] == _lib.MLA_ERR_INVALID_ARG
    assert sel(scores=None)[0] == _lib.MLA_ERR_INVALID_ARG
    assert sel(topk_idx=None)[0] == _lib.MLA_ERR_INVALID_ARG
    assert sel(scores=_P(FAKE + 4))[0] == _lib.MLA_ERR_INVALID_ARG
    assert sel(T=0)[0] == 0


def test_partition_validation_errors():
    f = _P(FAKE)
    p = lambda **kw: _status(lambda: _lib.pcp_partition(**{**dict(
        q_lens=_Len(2, FAKE), kv_lens=f, kv_start=f, P=2, T_glob=10, n_vrows=3, T_loc_total=10,
        cu_seqlens_glob=f, cu_seqlens_q=f, vrow_req=f, vrow_kv_start=f, vrow_kv_len=f, local_gidx=f,
        positions=f, slot=f, merge_src=f, stream=0), **kw}))
    assert p(P=0)[0] == _lib.MLA_ERR_INVALID_ARG
    assert p(n_vrows=5)[0] == _lib.MLA_ERR_INVALID_ARG  # more than 2 per request
    assert p(n_vrows=1)[0] == _lib.MLA_ERR_INVALID_ARG  # fewer than 1 per request
    assert p(merge_src=None)[0] == _lib.MLA_ERR_INVALID_ARG
    assert p(T_glob=-1)[0] == _lib.MLA_ERR_INVALID_ARG
    assert p(block_table=f, bt_stride=0)[0] == _lib.MLA_ERR_INVALID_ARG


class _Len(_P):
    def __init__(self, n, addr):
        super().__init__(addr)
        self.n = n

    def numel(self):
        return self.n


def test_merge_rejects_too_many_heads():
    f = _P(FAKE)
    st, _ = _status(lambda: _lib.pcp_lse_merge(f, f, f, 2, 4, 129, 64, 8, None, f, None, stream=0))
    assert st == _lib.MLA_ERR_UNSUPPORTED


def test_binding_rejects_buffers_smaller_than_the_call():
    """The binding checks each tensor's bytes (to the end of its storage, so views into a
    larger buffer pass) against what the call reads or writes, before the library runs: fp8
    codes (one byte per element) handed to the fp8 insert, which reads bf16 rows, are refused."""
    import torch
    T, Dl, Dr, N = 8, 512, 64, 64
    codes = torch.zeros(T, Dl, dtype=torch.uint8)
    rope = torch.zeros(T, Dr, dtype=torch.bfloat16)
    slot = torch.zeros(T, dtype=torch.int32)
    kv = torch.zeros(N, Dl, dtype=torch.uint8)
    kv_rope = torch.zeros(N, Dr, dtype=torch.bfloat16)
    scale = torch.zeros(1, dtype=torch.float32)
    with pytest.raises(_lib.MlaError, match="local_latent"):
        _lib.pcp_kv_insert_fp8(codes, rope, slot, T, Dl, Dr, N, kv, kv_rope, scale, stream=0)
    # a view: its storage runs past the view, which is what a kernel writing later split
    # slices through the view's pointer relies on
    big = torch.zeros(4 * T, 16, Dl, dtype=torch.bfloat16)
    _lib._need(big[T:2 * T], 3 * T * 16 * Dl * 2, "view")
    with pytest.raises(_lib.MlaError):
        _lib._need(big[T:2 * T], 3 * T * 16 * Dl * 2 + 2, "view")
