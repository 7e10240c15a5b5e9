"""Writing new tokens into the paged caches, and the e4m3 query cast.

Test infrastructure only (see the package docstring).

This is the step in front of the decode path (ROCm/ATOM PR 2962, the commit
messages under Follow-ups: one fused kernel encodes the new tokens' keys and
values in the MXFP4 / fp8 page format and emits the query in float8_e4m3fn,
scale 1, clamped at the format's maximum).  Readings where the sources are silent:

* placement - token i of request r's q new tokens sits at absolute position
  seq_lens[r] - q + i (the lengths include the new tokens); a position below
  zero (a pad request) is not written;
* e4m3fn encoding with a per-tensor scale - the library's quantiser is
  defined on its own interface: the scale is an fp32 argument and the value an
  fp32 number (bf16 inputs, or the fp32 result of the optional norm / rope), so
  the quotient is the fp32 division fl32(x / scale), and the code is that
  quotient rounded to the nearest e4m3fn value, ties to the even code -
  exactly what the plain tensor expression (x / scale).to(float8_e4m3fn)
  computes on fp32 tensors.  Magnitudes above 448 saturate to 448 (the
  saturating cast of ROCm/ATOM PR 2962, Follow-ups), NaN becomes 0x7F and the
  sign is kept (a negative value that rounds to zero is -0), as in every
  encoding here.  Rounding the fp32 quotient can differ from rounding the exact
  quotient where the two lie on either side of a midpoint between two codes;
  this definition takes the fp32 quotient.  With a unit scale (the query
  cast) the quotient is exact and the two agree;
* MXFP4 encoding (OCP MX v1.0) - per 32 consecutive dims the shared exponent
  is floor(log2 amax) - 2 (2 is the largest e2m1 exponent), clamped to the
  e8m0 range [-127, 127] (-127 for an all-zero group); each element's e2m1
  code rounds x / 2^exponent to nearest, ties to the even code, and magnitudes
  above 6 saturate to 6;
* bf16 values are stored as given;
* a layer that reuses another layer's top-k has no index key to write: the
  writer then takes no index vector and leaves the index pool alone;
* QK-norm and rope (optional, per vector kind: K, index key, query) - the
  pages name the fused QK-norm / rope step but none of its parameters, so the
  caller supplies them: RMS normalisation of each 128-dim head vector,
  y_d = w_d x_d / sqrt(mean(x^2) + eps), then the rotation of dim pairs
  (a, b) -> (a cos - b sin, b cos + a sin) at the token's position p, with
  cos / sin read from the caller's tables [positions][rot_dim / 2]; pairs are
  (i, i + rot_dim / 2) (NeoX) or (2i, 2i + 1) (interleaved), dims past rot_dim
  are left alone.  V is stored as given.  The transformed value is rounded to
  fp32 (the kernel's precision) before it is encoded; bf16 storage rounds to
  nearest, ties to even.

Every code below is chosen from the decoded value tables of ``formats`` (the
nearest representable value, ties to the even code), and bytes are placed with
the page offset formulas of ``pools``, so the writer is the exact inverse of the
readers the oracle's decode path uses.
"""
from __future__ import annotations

import numpy as np

from . import formats, pools

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _nearest_code(a: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of the increasing table to each a >= 0 (a
    within the table's range), ties to the even index."""
    hi = np.clip(np.searchsorted(table, a, side="left"), 1, len(table) - 1)
    lo = hi - 1
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


_E4M3_TABLE = np.array([formats.e4m3_value(c) for c in range(0x7F)])   # codes 0x00..0x7E, increasing
_E2M1_TABLE = np.array([formats.e2m1_value(c) for c in range(8)])      # 0, .5, 1, 1.5, 2, 3, 4, 6


def encode_e4m3(x) -> np.ndarray:
    """e4m3fn bytes of x (any shape), rounding and saturating as above."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = _nearest_code(np.where(np.isnan(a), 0.0, a), _E4M3_TABLE).astype(np.uint8)
    code = code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def encode_e2m1(x) -> np.ndarray:
    """4-bit e2m1 codes of x (finite), rounding and saturating as above."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    code = _nearest_code(a, _E2M1_TABLE).astype(np.uint8)
    return code | np.where(np.signbit(x), 8, 0).astype(np.uint8)


def mx_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """x [..., 128] -> (e2m1 codes [..., 128], e8m0 scale bytes [..., 4])."""
    x = np.asarray(x, dtype=np.float64)
    g = x.reshape(*x.shape[:-1], 4, 32)
    amax = np.abs(g).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127.0)
    e = np.clip(e, -127, 127)
    codes = encode_e2m1(g / np.exp2(e)[..., None]).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def _mxfp4_put(flat: np.ndarray, base: int, slot: int, codes: np.ndarray, scales: np.ndarray) -> None:
    """Token `slot` of the 8704 B MXFP4 page at byte `base` of a flat pool
    (formats.decode_mxfp4_page's layout)."""
    flat[base + 64 * slot:base + 64 * slot + 64] = codes[0::2] | (codes[1::2] << 4)
    s0 = base + formats.MXFP4_DATA_BYTES + 4 * slot
    flat[s0:s0 + 4] = scales


def bf16_bits(x) -> np.ndarray:
    """bf16 codes of x (rounded to fp32 first): round to nearest, ties to even;
    NaN becomes a quiet NaN with its sign."""
    u = np.asarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    rne = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = ((u & 0x7FFFFFFF) > 0x7F800000)
    return np.where(nan, (u >> 16) | 0x40, rne).astype(np.uint16)


def _bf16_bytes(x: np.ndarray) -> np.ndarray:
    """values -> the two bytes of each one's bf16 code (the identity on bf16 values)."""
    return bf16_bits(x).view(np.uint8).reshape(*np.shape(x), 2)


def rms_norm(x, weight, eps: float) -> np.ndarray:
    """x [..., 128] -> w * x / sqrt(mean(x^2) + eps), per vector."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(weight, dtype=np.float64) * x / np.sqrt(ms + eps)


def rope(x, pos: int, cos, sin, rot_dim: int, neox: bool) -> np.ndarray:
    """One 128-dim vector rotated at position pos: pair i of the first rot_dim
    dims turns by the angle whose cosine / sine are cos[pos][i] / sin[pos][i]."""
    y = np.array(x, dtype=np.float64)
    half = rot_dim // 2
    c = np.asarray(cos, dtype=np.float64)[pos, :half]
    s_ = np.asarray(sin, dtype=np.float64)[pos, :half]
    if neox:
        a, b = y[:half].copy(), y[half:rot_dim].copy()
        y[:half], y[half:rot_dim] = a * c - b * s_, b * c + a * s_
    else:
        a, b = y[0:rot_dim:2].copy(), y[1:rot_dim:2].copy()
        y[0:rot_dim:2], y[1:rot_dim:2] = a * c - b * s_, b * c + a * s_
    return y


def transform(x, pos: int, tf) -> np.ndarray:
    """The optional QK-norm then rope of one vector; tf is None or a dict with
    norm_weight (None: no norm), eps, cos / sin (None: no rope), rot_dim, neox.
    Rounded to fp32, the precision the stored value is decided in."""
    y = np.asarray(x, dtype=np.float64)
    if tf is not None:
        if tf.get("norm_weight") is not None:
            y = rms_norm(y, tf["norm_weight"], tf["eps"])
        if tf.get("cos") is not None:
            y = rope(y, pos, tf["cos"], tf["sin"], tf["rot_dim"], tf["neox"])
    return y.astype(np.float32).astype(np.float64)


def quantize_e4m3_scaled(x, scale: float) -> np.ndarray:
    """e4m3fn bytes of the fp32 quotient fl32(x / scale): x and scale are fp32
    numbers (x rounded to fp32 first), the division is IEEE fp32 division,
    then encode_e4m3 rounds that quotient (see the module docstring)."""
    y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return encode_e4m3(y.astype(np.float64))


def _element_bytes(x: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """[..., 128] values -> [..., 128, e] stored bytes for bf16 / fp8."""
    if dtype == "bf16":
        return _bf16_bytes(x)
    return quantize_e4m3_scaled(x, scale)[..., None]


def write_cache(k_new, v_new, idx_new, block_table, seq_lens, q_len: int,
                k_pool: np.ndarray, v_pool: np.ndarray, kv_dtype: str, k_scale: float, v_scale: float,
                idx_pool: np.ndarray, idx_dtype: str, idx_scale: float, k_tf=None, idx_tf=None) -> None:
    """Writes the new tokens into the pools, in place.

    k_new, v_new [T, H_kv, 128] and idx_new [T, 128] (or None: no index key)
    hold the values (floats; bf16 caches take values that bf16 represents
    exactly); the pools are the
    contiguous byte arrays the readers of ``pools`` take (K/V: pages of
    H_kv heads each, head g of page id n at (n H_kv + g) page bytes; index
    cache: one page per block).  k_tf / idx_tf: the optional QK-norm and rope
    of the keys and of the index keys (see ``transform``)."""
    T, H_kv, _ = np.shape(k_new)
    with_idx = idx_new is not None
    k_new, v_new = (np.asarray(a, dtype=np.float64) for a in (k_new, v_new))
    kf, vf = (np.asarray(a).reshape(-1) for a in (k_pool, v_pool))  # flat byte views
    assert np.shares_memory(kf, k_pool) and np.shares_memory(vf, v_pool)
    if with_idx:
        idx_new = np.asarray(idx_new, dtype=np.float64)
        xf = np.asarray(idx_pool).reshape(-1)
        assert np.shares_memory(xf, idx_pool)
    for t in range(T):
        r, i = divmod(t, q_len)
        p = int(seq_lens[r]) - q_len + i
        if p < 0:
            continue
        blk, slot = int(block_table[r][p // pools.BLOCK]), p % pools.BLOCK
        kt = [transform(k_new[t, g], p, k_tf) for g in range(H_kv)]
        it = transform(idx_new[t], p, idx_tf) if with_idx else None
        # index key: one per token, no head dimension; page id = block id
        if not with_idx:
            pass
        elif idx_dtype == "mxfp4":
            codes, scales = mx_quantize(it)
            _mxfp4_put(xf, blk * formats.MXFP4_PAGE_BYTES, slot, codes, scales)
        else:
            e = 2 if idx_dtype == "bf16" else 1
            off = blk * 16384 * e + 2048 * e * (slot // pools.PAGE16) + _k_offsets_row(e, slot % pools.PAGE16)
            xf[off] = _element_bytes(it, idx_dtype, idx_scale).reshape(-1)
        for g in range(H_kv):
            if kv_dtype == "mxfp4":
                for flat, x in ((kf, kt[g]), (vf, v_new[t, g])):
                    codes, scales = mx_quantize(x)
                    _mxfp4_put(flat, (blk * H_kv + g) * formats.MXFP4_PAGE_BYTES, slot, codes, scales)
            else:
                e = 2 if kv_dtype == "bf16" else 1
                base = ((8 * blk + slot // pools.PAGE16) * H_kv + g) * 2048 * e
                c = slot % pools.PAGE16
                kf[base + _k_offsets_row(e, c)] = _element_bytes(kt[g], kv_dtype, k_scale).reshape(-1)
                vf[base + _v_offsets_row(e, c)] = _element_bytes(v_new[t, g], kv_dtype, v_scale).reshape(-1)


def _k_offsets_row(esize: int, c: int) -> np.ndarray:
    """Byte offsets of the 128 dims of key c of a 16-token K page, each element's bytes in order."""
    return (pools._k_offsets(esize)[c][:, None] + np.arange(esize)).reshape(-1)


def _v_offsets_row(esize: int, t: int) -> np.ndarray:
    """Byte offsets of the 128 dims of key t of a 16-token V page, each element's bytes in order."""
    return (pools._v_offsets(esize)[t][:, None] + np.arange(esize)).reshape(-1)


def quantize_query_e4m3(q) -> np.ndarray:
    """The query cast of the fused writer: e4m3fn bytes with a unit scale, saturating."""
    return encode_e4m3(q)


def prepare_query(q, seq_lens, q_len: int, tf, out_dtype: str) -> np.ndarray:
    """Queries [T, H, 128] of the step's tokens: the optional QK-norm and rope
    at each token's position, then stored as bf16 codes (uint16) or unit-scale
    e4m3 codes (uint8).  Rows of pad tokens (position < 0) are zero."""
    q = np.asarray(q, dtype=np.float64)
    T, H, _ = q.shape
    out = np.zeros((T, H, 128), dtype=np.uint16 if out_dtype == "bf16" else np.uint8)
    for t in range(T):
        r, i = divmod(t, q_len)
        p = int(seq_lens[r]) - q_len + i
        if p < 0:
            continue
        for h in range(H):
            y = transform(q[t, h], p, tf)
            out[t, h] = bf16_bits(y) if out_dtype == "bf16" else encode_e4m3(y)
    return out
