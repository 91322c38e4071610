"""Exact number decoding for the oracle (test infrastructure only).

* bf16: the top 16 bits of an IEEE binary32; decoding is exact in fp64.
* bf16 round-to-nearest-even of an fp32 value: used only to reproduce the one
  rounding the kernel applies to dequantised fp8 KV before the MFMA (a reading:
  the pages name an fp8 MLA cache, "[Feature][PCP] Add DeepSeek-V4.1-Flash support",
  "vLLM Launch Arguments", without its layout).
* OCP OFP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
  subnormals, no infinities, S.1111.111 = NaN; largest finite value 448.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to the nearest bfloat16 (ties to even); returns float64.

    Written from the definition: keep the top 16 bits, and round up when the
    dropped 16 bits exceed half an ulp, or equal half an ulp with an odd kept part.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    kept = u >> np.uint64(16)
    dropped = u & np.uint64(0xFFFF)
    up = (dropped > 0x8000) | ((dropped == 0x8000) & ((kept & np.uint64(1)) == 1))
    kept = kept + up.astype(np.uint64)
    return bf16_to_f64((kept & np.uint64(0xFFFF)).astype(np.uint16))


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes (uint8) -> float64 by the format's formula."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    subnormal = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


def dequant_fp8_rows(codes: np.ndarray, row_ids: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Latent rows from fp8 codes: bf16_rne(fp32(decode(code) * scale[row // 64])).

    ``row_ids`` are the packed KV rows of ``codes``; the tile scale of row r is
    ``scales[r // 64]``. The product is taken in binary32, as the kernel does.
    """
    v = e4m3fn_decode(codes).astype(np.float32)  # exact: 4 significant bits
    s = np.asarray(scales, dtype=np.float32)[np.asarray(row_ids) // 64]
    prod = (v * s[:, None]).astype(np.float32)  # one binary32 rounding
    return f32_to_bf16_rne(prod)


def _e4m3fn_magnitudes() -> np.ndarray:
    """Values of the finite non-negative codes 0x00..0x7E, in code order (increasing)."""
    return e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3fn_encode_rne(x: np.ndarray) -> np.ndarray:
    """Nearest OCP E4M3FN code of each binary32 value in [-448, 448] (ties to the even
    code, i.e. mantissa LSB 0); the sign bit follows the sign of x, -0.0 included.

    The finite magnitudes are increasing in code order, so the nearest one is one of the
    two that bracket |x|; of two at the same distance the even code wins (round to
    nearest even). Values outside [-448, 448] or NaN are rejected: the caller clamps.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    if np.any(~(a <= 448.0)):
        raise ValueError("e4m3fn_encode_rne takes finite values in [-448, 448]")
    mags = _e4m3fn_magnitudes()
    hi = np.searchsorted(mags, a, side="left")  # first magnitude >= |x|
    hi = np.minimum(hi, len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
