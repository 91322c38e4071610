"""Paged latent-KV addressing and fp8 quantise-on-insert, written from their definitions
(oracle; test infrastructure only).

* Paged KV: the cache is a pool of 64-row blocks ("[Feature][PCP] Add DeepSeek-V4.1-Flash
  support", "vLLM Launch Arguments": KV cache block size 64). Request b's key at position
  j lives in row block_table[b][j // 64] * 64 + j % 64. With the identity table of a
  64-aligned packed layout this is the packed row kv_start[b] + j.
* fp8 MLA cache ("[Feature][PCP] Add DeepSeek-V4.1-Flash support", "vLLM Launch
  Arguments": fp8 MLA KV cache): OCP E4M3FN latent codes with one fp32 scale per 64-row
  block, rope kept bf16. The pages name the cache but not its layout; the reading taken
  here is a power-of-two block scale, the smallest one not below a / 448 with a the
  block's largest |x| (shared power-of-two scales as in the OCP microscaling formats),
  set by the insert that writes the block's first row, later rows of the block quantised
  against that stored scale with saturation at +-448.
"""
import numpy as np

from . import numerics as on

BLOCK = 64
E4M3_MAX = 448.0


def paged_rows(block_table: np.ndarray, b: int, positions: np.ndarray) -> np.ndarray:
    """Cache rows of request b's keys at the given positions."""
    pos = np.asarray(positions, dtype=np.int64)
    return np.asarray(block_table, dtype=np.int64)[b, pos // BLOCK] * BLOCK + pos % BLOCK


def pow2_at_least(r) -> np.float32:
    """The smallest power of two 2^e >= r with e >= -126 (normal binary32), for r >= 0."""
    r = float(np.float32(r))
    e = -126
    while 2.0 ** e < r:
        e += 1
    return np.float32(2.0 ** e)


def quantize_insert_fp8(codes: np.ndarray, scales: np.ndarray, lat_bits: np.ndarray, slot: np.ndarray):
    """One quantise-on-insert call. Returns new (codes, scales); the inputs are not changed.

    codes   uint8 [N_kv, D] cache latent codes before the call;
    scales  float32 [ceil(N_kv / 64)] block scales before the call;
    lat_bits bf16 bit patterns [T, D] of the rows written;
    slot    int [T] destination rows (rows outside [0, N_kv) are skipped).

    Steps: (1) the blocks this call opens are those of slots s with s % 64 == 0;
    (2) for each, a = max |x| over the elements the call writes into it, and its scale
    becomes pow2_at_least(fp32(a / 448)), or 1 when a == 0; (3) each written element
    becomes e4m3fn_rne(clamp(fp32(x / scale), -448, 448)) with its block's scale (new or
    stored).
    """
    codes = np.array(codes, dtype=np.uint8, copy=True)
    scales = np.array(scales, dtype=np.float32, copy=True)
    N_kv = codes.shape[0]
    slot = np.asarray(slot, dtype=np.int64)
    keep = (slot >= 0) & (slot < N_kv)
    rows = np.nonzero(keep)[0]
    s = slot[rows]
    x = on.bf16_to_f64(np.asarray(lat_bits)[rows]).astype(np.float32)  # exact
    blk = s // BLOCK
    opened = np.unique(blk[s % BLOCK == 0])
    for B in opened:
        a = np.float32(np.max(np.abs(x[blk == B]))) if np.any(blk == B) else np.float32(0.0)
        scales[B] = pow2_at_least(np.float32(a) / np.float32(E4M3_MAX)) if a > 0 else np.float32(1.0)
    sc = scales[blk][:, None]
    y = np.clip((x / sc).astype(np.float32), -E4M3_MAX, E4M3_MAX)
    codes[s] = on.e4m3fn_encode_rne(y)
    return codes, scales
