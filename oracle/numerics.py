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
