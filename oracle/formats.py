"""Exact decoding of the cache element formats, in float64.

Test infrastructure only (see the package docstring).

Formats, as the sources name them:
* e4m3fn - ``float8_e4m3fn`` K/V and index values and the e4m3 query
  (ROCm/ATOM PR 2962, Summary: the MXFP4 index is scored with an e4m3 index
  query; the fused-writer commit message: the query emitted in
  ``float8_e4m3fn`` with scale 1, clamped at the format's maximum).
  Definition (OCP 8-bit floating point, E4M3): sign s, 4 exponent bits E
  (bias 7), 3 mantissa bits m; E = 0 is subnormal 2^-6 * m/8; all other codes
  are 2^(E-7) * (1 + m/8) except E = 15, m = 7, which is NaN; no infinities.
* e2m1 - the MXFP4 element (PR 2962, Summary: the data part of a page).  OCP MX v1.0:
  sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6.
* e8m0 - the MXFP4 block scale, one per 32 elements (PR 2962, Summary).
  OCP MX v1.0: 2^(E - 127); E = 255 is NaN.
* bf16 - the top 16 bits of an IEEE binary32.
"""
from __future__ import annotations

import numpy as np

MXFP4_DATA_BYTES = 128 * 64      # 128 tokens x 64 B of e2m1 data
MXFP4_SCALE_BYTES = 128 * 4      # 128 tokens x 4 e8m0 scales
MXFP4_PAGE_BYTES = MXFP4_DATA_BYTES + MXFP4_SCALE_BYTES


def e4m3_value(code: int) -> float:
    """Value of one e4m3fn byte, from the definition (slow, scalar)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        v = 2.0 ** -6 * (m / 8.0)
    else:
        v = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -v if s else v


def e2m1_value(code: int) -> float:
    """Value of one 4-bit e2m1 code, from the definition (slow, scalar)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        v = 0.5 * m
    else:
        v = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -v if s else v


def e8m0_value(code: int) -> float:
    """Value of one e8m0 scale byte: 2^(code - 127); 255 is NaN."""
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


# Per-code tables built from the scalar definitions above; the vector decoders
# below only index them.
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(b: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(b, dtype=np.uint8)]


def decode_e2m1(nib: np.ndarray) -> np.ndarray:
    return E2M1_TABLE[np.asarray(nib, dtype=np.uint8) & 0xF]


def decode_e8m0(b: np.ndarray) -> np.ndarray:
    return E8M0_TABLE[np.asarray(b, dtype=np.uint8)]


def decode_bf16_bytes(b: np.ndarray) -> np.ndarray:
    """Little-endian bf16 byte pairs [..., 2n] -> float64 [..., n]."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8))
    u16 = b.view(np.uint16).astype(np.uint32)
    with np.errstate(invalid="ignore"):          # signalling-NaN codes stay NaN
        return (u16 << 16).view(np.float32).astype(np.float64)


def decode_query(b: np.ndarray, dtype: str) -> np.ndarray:
    """Query rows stored as raw bytes [..., 128 * esize] -> float64 [..., 128]."""
    if dtype == "bf16":
        return decode_bf16_bytes(b)
    if dtype == "e4m3":
        return decode_e4m3(b)
    raise ValueError(dtype)


def decode_mxfp4_page(page: np.ndarray) -> np.ndarray:
    """One or more 8704 B MXFP4 pages [..., 8704] -> float64 [..., 128 tokens, 128 dims].

    Page format (PR 2962, Summary and the commit that declares the MXFP4 caches):
    128 x 64 B of e2m1 data, then 128 x 4 B of e8m0 scales.  Readings where the
    sources are silent: token j's data at byte 64 j and its scales at byte
    8192 + 4 j; dim 2c in the low nibble of byte c and dim 2c+1 in the high
    nibble (the OCP MX packing order); scale s covers dims 32 s .. 32 s + 31.
    """
    page = np.asarray(page, dtype=np.uint8)
    assert page.shape[-1] == MXFP4_PAGE_BYTES
    lead = page.shape[:-1]
    data = page[..., :MXFP4_DATA_BYTES].reshape(*lead, 128, 64)
    scales = page[..., MXFP4_DATA_BYTES:].reshape(*lead, 128, 4)
    lo = decode_e2m1(data & 0xF)
    hi = decode_e2m1(data >> 4)
    vals = np.empty((*lead, 128, 128), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    sc = decode_e8m0(scales)                       # [..., 128, 4]
    return vals * np.repeat(sc, 32, axis=-1)
