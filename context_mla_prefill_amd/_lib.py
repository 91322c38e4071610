"""ctypes binding of ``libmla_pcp.so`` (the C ABI in ``include/mla_pcp.h``).

Argument marshalling only: every function here has the name of a C entry point, turns
torch tensors into device pointers and the current torch stream into a hipStream_t,
and raises ``MlaError`` on a non-OK status. All computation runs in the library's HIP
kernels; there is no fallback. Importing this module loads nothing; the first call
(or :func:`load`) loads the in-tree library and fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_pcp.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP = 0, 1, 2, 3
MLA_KV_BF16, MLA_KV_FP8_E4M3 = 0, 1
ABI_VERSION = 6

EXPORTED = ("mla_pcp_abi_version", "mla_pcp_last_error", "pcp_plan_sizes", "pcp_partition",
            "pcp_kv_insert", "pcp_kv_insert_fp8", "pcp_kv_dequant_fp8", "sparse_topk_select", "mla_prefill_partial",
            "pcp_lse_merge", "pcp_plan_splits")

_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


class mla_partial_args(ctypes.Structure):
    _fields_ = [
        ("q", _p), ("latent_kv", _p), ("kv_scale", _p), ("rope_k", _p),
        ("cu_seqlens_q", _p), ("vrow_kv_start", _p), ("positions", _p), ("topk_idx", _p),
        ("topk", _i32), ("window", _i32), ("n_vrows", _i32), ("T_loc", _i32), ("H", _i32),
        ("D_latent", _i32), ("D_rope", _i32), ("kv_dtype", _i32), ("N_kv", _i64),
        ("scale", ctypes.c_float), ("o_partial", _p), ("lse", _p),
        ("kv_splits", _i32), ("split_stride", _i64), ("vrow_kv_len", _p),
        ("block_table", _p), ("bt_stride", _i32), ("vrow_req", _p),
        ("vrow_splits", _p), ("vrow_order", _p),
    ]


def load():
    """Load the built library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run __graft_entry__.build() or python -m context_mla_prefill_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mla_pcp_abi_version.restype = ctypes.c_int
    lib.mla_pcp_abi_version.argtypes = []
    lib.mla_pcp_last_error.restype = ctypes.c_char_p
    lib.mla_pcp_last_error.argtypes = []
    lib.pcp_plan_sizes.restype = ctypes.c_int
    lib.pcp_plan_sizes.argtypes = [_pi32, _pi32, _i32, _i32, _pi32, _pi32, _pi64]
    lib.pcp_partition.restype = ctypes.c_int
    lib.pcp_partition.argtypes = [_p, _p, _p, _i32, _i32, _i64, _i32, _i64, _p, _i32, _p, _p, _p, _p, _p,
                                  _p, _p, _p, _p, _p]
    lib.pcp_kv_insert.restype = ctypes.c_int
    lib.pcp_kv_insert.argtypes = [_p, _p, _p, _i32, _i32, _i32, _i32, _i64, _p, _p, _p]
    lib.pcp_kv_insert_fp8.restype = ctypes.c_int
    lib.pcp_kv_insert_fp8.argtypes = [_p, _p, _p, _i32, _i32, _i32, _i64, _p, _p, _p, _p]
    lib.pcp_kv_dequant_fp8.restype = ctypes.c_int
    lib.pcp_kv_dequant_fp8.argtypes = [_p, _p, _i64, _i32, _p, _i32, _p, _p]
    lib.sparse_topk_select.restype = ctypes.c_int
    lib.sparse_topk_select.argtypes = [_p, _i64, _p, _i32, _i32, _p, _p]
    lib.mla_prefill_partial.restype = ctypes.c_int
    lib.mla_prefill_partial.argtypes = [ctypes.POINTER(mla_partial_args), _p]
    lib.pcp_lse_merge.restype = ctypes.c_int
    lib.pcp_plan_splits.argtypes = [_pi32, _pi32, _i32, _i32, _i32, _i32, _i32, _i32, _pi32, _pi32]
    lib.pcp_plan_splits.restype = ctypes.c_int
    lib.pcp_lse_merge.argtypes = [_p, _p, _p, _i32, _i64, _i32, _i32, _i64, _i32, _i64, _p, _p, _p, _p]
    if lib.mla_pcp_abi_version() != ABI_VERSION:
        raise RuntimeError(f"ABI mismatch: library {lib.mla_pcp_abi_version()} binding {ABI_VERSION}")
    _lib = lib
    return lib


def last_error() -> str:
    return load().mla_pcp_last_error().decode()


def _check(status: int, name: str):
    if status != MLA_OK:
        raise MlaError(status, f"{name}: {last_error()}")


def _ptr(t):
    """Device (or host) address of a tensor / numpy array, or NULL for None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _need(t, nbytes: int, what: str):
    """A tensor / array handed to the library must hold at least the bytes the call will
    touch (the C ABI takes bare pointers and cannot check this itself)."""
    if t is None or nbytes <= 0:
        return
    if isinstance(t, np.ndarray):
        have = t.nbytes
    elif hasattr(t, "untyped_storage"):  # bytes from the first element to the end of the storage
        st = t.untyped_storage()
        have = st.nbytes() - (t.data_ptr() - st.data_ptr())
    else:  # a bare address: its size is the caller's to guarantee
        return
    if have < nbytes:
        raise MlaError(MLA_ERR_INVALID_ARG, f"{what}: holds {have} bytes, the call reads or writes {nbytes}")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def mla_pcp_abi_version() -> int:
    return load().mla_pcp_abi_version()


def pcp_plan_sizes(q_lens, kv_lens, P: int):
    """Host sizing: returns (T_loc list[P], n_vrows, T_glob)."""
    lib = load()
    q = np.ascontiguousarray(q_lens, dtype=np.int32)
    kv = np.ascontiguousarray(kv_lens, dtype=np.int32)
    T_loc = np.zeros(max(P, 1), dtype=np.int32)
    nv = ctypes.c_int32(0)
    tg = ctypes.c_int64(0)
    st = lib.pcp_plan_sizes(q.ctypes.data_as(_pi32), kv.ctypes.data_as(_pi32), len(q), P,
                            T_loc.ctypes.data_as(_pi32), ctypes.byref(nv), ctypes.byref(tg))
    _check(st, "pcp_plan_sizes")
    return [int(x) for x in T_loc[:P]], int(nv.value), int(tg.value)


def pcp_plan_splits(q_lens, kv_lens, P: int, H: int, D_latent: int, max_splits: int, n_workers: int):
    """Host split-KV plan for the dense partials: (vrow_splits, vrow_order), int32 [P][n_vrows]."""
    lib = load()
    q = np.ascontiguousarray(q_lens, dtype=np.int32)
    kv = np.ascontiguousarray(kv_lens, dtype=np.int32)
    _, n_vrows, _ = pcp_plan_sizes(q, kv, P)
    splits = np.zeros((P, max(n_vrows, 1)), dtype=np.int32)
    order = np.zeros((P, max(n_vrows, 1)), dtype=np.int32)
    st = lib.pcp_plan_splits(q.ctypes.data_as(_pi32), kv.ctypes.data_as(_pi32), len(q), P, H, D_latent, max_splits,
                             n_workers, splits.ctypes.data_as(_pi32), order.ctypes.data_as(_pi32))
    _check(st, "pcp_plan_splits")
    return splits[:, :n_vrows], order[:, :n_vrows]


def pcp_partition(q_lens, kv_lens, kv_start, P, T_glob, n_vrows, T_loc_total, cu_seqlens_glob,
                  cu_seqlens_q, vrow_req, vrow_kv_start, vrow_kv_len, local_gidx, positions, slot,
                  merge_src, stream=None, block_table=None, bt_stride=0):
    st = load().pcp_partition(_ptr(q_lens), _ptr(kv_lens), _ptr(kv_start), int(q_lens.numel()), P,
                              T_glob, n_vrows, T_loc_total, _ptr(block_table), bt_stride,
                              _ptr(cu_seqlens_glob), _ptr(cu_seqlens_q),
                              _ptr(vrow_req), _ptr(vrow_kv_start), _ptr(vrow_kv_len), _ptr(local_gidx),
                              _ptr(positions), _ptr(slot), _ptr(merge_src), _stream(stream))
    _check(st, "pcp_partition")


def pcp_kv_insert(local_latent, local_rope, slot, T_loc, D_latent, D_rope, kv_dtype, N_kv, kv_latent,
                  kv_rope, stream=None):
    eb = 2 if kv_dtype == MLA_KV_BF16 else 1
    _need(local_latent, T_loc * D_latent * eb, "pcp_kv_insert local_latent")
    _need(local_rope, T_loc * D_rope * 2, "pcp_kv_insert local_rope")
    _need(slot, T_loc * 4, "pcp_kv_insert slot")
    _need(kv_latent, N_kv * D_latent * eb, "pcp_kv_insert kv_latent")
    _need(kv_rope, N_kv * D_rope * 2, "pcp_kv_insert kv_rope")
    st = load().pcp_kv_insert(_ptr(local_latent), _ptr(local_rope), _ptr(slot), T_loc, D_latent, D_rope,
                              kv_dtype, N_kv, _ptr(kv_latent), _ptr(kv_rope), _stream(stream))
    _check(st, "pcp_kv_insert")


def pcp_kv_insert_fp8(local_latent, local_rope, slot, T, D_latent, D_rope, N_kv, kv_latent, kv_rope, kv_scale,
                      stream=None):
    _need(local_latent, T * D_latent * 2, "pcp_kv_insert_fp8 local_latent (bf16 rows)")
    _need(local_rope, T * D_rope * 2, "pcp_kv_insert_fp8 local_rope")
    _need(slot, T * 4, "pcp_kv_insert_fp8 slot")
    _need(kv_latent, N_kv * D_latent, "pcp_kv_insert_fp8 kv_latent")
    _need(kv_rope, N_kv * D_rope * 2, "pcp_kv_insert_fp8 kv_rope")
    _need(kv_scale, (N_kv + 63) // 64 * 4, "pcp_kv_insert_fp8 kv_scale")
    st = load().pcp_kv_insert_fp8(_ptr(local_latent), _ptr(local_rope), _ptr(slot), T, D_latent, D_rope, N_kv,
                                  _ptr(kv_latent), _ptr(kv_rope), _ptr(kv_scale), _stream(stream))
    _check(st, "pcp_kv_insert_fp8")


def pcp_kv_dequant_fp8(kv_latent, kv_scale, N_kv, D_latent, blocks, n_blocks, ws, stream=None):
    _need(kv_latent, N_kv * D_latent, "pcp_kv_dequant_fp8 kv_latent")
    _need(kv_scale, (N_kv + 63) // 64 * 4, "pcp_kv_dequant_fp8 kv_scale")
    _need(blocks, n_blocks * 4, "pcp_kv_dequant_fp8 blocks")
    _need(ws, N_kv * D_latent * 2, "pcp_kv_dequant_fp8 ws")
    st = load().pcp_kv_dequant_fp8(_ptr(kv_latent), _ptr(kv_scale), N_kv, D_latent, _ptr(blocks), n_blocks, _ptr(ws),
                                   _stream(stream))
    _check(st, "pcp_kv_dequant_fp8")


def sparse_topk_select(scores, ld, positions, T, k, topk_idx, stream=None):
    _need(positions, T * 4, "sparse_topk_select positions")
    _need(topk_idx, T * k * 4, "sparse_topk_select topk_idx")
    st = load().sparse_topk_select(_ptr(scores), ld, _ptr(positions), T, k, _ptr(topk_idx), _stream(stream))
    _check(st, "sparse_topk_select")


def make_partial_args(q, latent_kv, rope_k, cu_seqlens_q, vrow_kv_start, positions, n_vrows, T_loc, H,
                      D_latent, D_rope, scale, o_partial, lse, N_kv, kv_dtype=MLA_KV_BF16, kv_scale=None,
                      topk_idx=None, topk=0, window=0, kv_splits=1, split_stride=0,
                      vrow_kv_len=None, block_table=None, bt_stride=0, vrow_req=None, vrow_splits=None,
                      vrow_order=None) -> mla_partial_args:
    rows = (split_stride * (kv_splits - 1) + T_loc) if kv_splits > 1 else T_loc
    eb = 2 if kv_dtype == MLA_KV_BF16 else 1
    _need(q, T_loc * H * (D_latent + D_rope) * 2, "mla_prefill_partial q")
    _need(latent_kv, N_kv * D_latent * eb, "mla_prefill_partial latent_kv")
    _need(rope_k, N_kv * D_rope * 2, "mla_prefill_partial rope_k")
    _need(positions, T_loc * 4, "mla_prefill_partial positions")
    _need(topk_idx, T_loc * topk * 4, "mla_prefill_partial topk_idx")
    _need(o_partial, rows * H * D_latent * 2, "mla_prefill_partial o_partial")
    _need(lse, rows * H * 4, "mla_prefill_partial lse")
    _need(cu_seqlens_q, (n_vrows + 1) * 4, "mla_prefill_partial cu_seqlens_q")
    _need(vrow_kv_start, n_vrows * 4, "mla_prefill_partial vrow_kv_start")
    _need(vrow_splits, n_vrows * 4, "mla_prefill_partial vrow_splits")
    _need(vrow_order, n_vrows * 4, "mla_prefill_partial vrow_order")
    if kv_dtype != MLA_KV_BF16:
        _need(kv_scale, (N_kv + 63) // 64 * 4, "mla_prefill_partial kv_scale")
    return mla_partial_args(
        q=_ptr(q), latent_kv=_ptr(latent_kv), kv_scale=_ptr(kv_scale), rope_k=_ptr(rope_k),
        cu_seqlens_q=_ptr(cu_seqlens_q), vrow_kv_start=_ptr(vrow_kv_start), positions=_ptr(positions),
        topk_idx=_ptr(topk_idx), topk=topk, window=window, n_vrows=n_vrows, T_loc=T_loc, H=H,
        D_latent=D_latent, D_rope=D_rope, kv_dtype=kv_dtype, N_kv=N_kv, scale=float(scale),
        o_partial=_ptr(o_partial), lse=_ptr(lse), kv_splits=kv_splits, split_stride=split_stride,
        vrow_kv_len=_ptr(vrow_kv_len), block_table=_ptr(block_table), bt_stride=bt_stride,
        vrow_req=_ptr(vrow_req), vrow_splits=_ptr(vrow_splits), vrow_order=_ptr(vrow_order))


def mla_prefill_partial(args: mla_partial_args, stream=None):
    st = load().mla_prefill_partial(ctypes.byref(args), _stream(stream))
    _check(st, "mla_prefill_partial")


def pcp_lse_merge(o_cat, lse_cat, merge_src, P, T_glob, H, D_v, R_total, sink, o_out, lse_out,
                  stream=None, kv_splits=1, split_stride=0):
    _need(o_cat, R_total * H * D_v * 2, "pcp_lse_merge o_cat")
    _need(lse_cat, R_total * H * 4, "pcp_lse_merge lse_cat")
    _need(merge_src, T_glob * P * 4, "pcp_lse_merge merge_src")
    _need(o_out, T_glob * H * D_v * 2, "pcp_lse_merge o_out")
    _need(lse_out, T_glob * H * 4, "pcp_lse_merge lse_out")
    _need(sink, H * 4, "pcp_lse_merge sink")
    st = load().pcp_lse_merge(_ptr(o_cat), _ptr(lse_cat), _ptr(merge_src), P, T_glob, H, D_v, R_total,
                              kv_splits, split_stride, _ptr(sink), _ptr(o_out), _ptr(lse_out), _stream(stream))
    _check(st, "pcp_lse_merge")
