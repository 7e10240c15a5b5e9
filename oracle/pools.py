"""Reading tokens out of the paged caches, in float64.

Test infrastructure only (see the package docstring).

Pool layout read here (its own code; it shares nothing with the GPU path):

* index cache - one page per 128-token block, page id = block id
  (ROCm/ATOM PR 2962, the commit that declares the MXFP4 caches: the index
  cache holds one 8704 B page for each 128-token block):
    bf16  eight 16-token tiles, each in the element order of a 16-token K
          page (below);
    fp8   the same with e4m3 elements, times the per-tensor ``idx_scale``
          (reading: the index cache takes one per-tensor scale, the same
          convention as the fp8 K/V cache);
    mxfp4 the 8704 B page of ``formats.decode_mxfp4_page``.
* K/V cache, bf16 / fp8 - 16-token pages, 8 per 128-token block
  (vLLM API page for ``sparse_attention_msa``: the page-16 rebase of the block
  table and the stride check over the pages of a sparse block).  Within a
  page the element order is this library's own (the sources show only that a
  16-token page is sub-tiled for the kernel, vLLM PR 61889, Validation, the
  K [.., 8, 16, 16] and V [.., 1, 128, 16] shapes).  With e = bytes per element:
    K: key c, dim d at byte 1024 ((d mod 32) div (16/e)) + 256 (d div 32)
       + 16 c + e (d mod (16/e));
    V: key t, dim d = 16 dt + c at byte 1024 (dt div (4/e)) + 256 (t div 4)
       + 16 c + 4 e (dt mod (4/e)) + e (t mod 4).
  fp8 values are multiplied by the per-tensor ``k_scale`` / ``v_scale``.  One
  page id addresses a K page and a V page (vLLM PR 61889, Details).
* K/V cache, mxfp4 - one 8704 B page per block for K and one for V
  (PR 2962, Summary: K and V use the same MXFP4 page format).
* A K/V page id holds one page per KV head ([num_pages][H_kv][page]): in the
  MXFP4 caches K and V each get a page for every pair of page id and KV head,
  while the index key gets one page for each block, whatever the head count
  (PR 2962, the commit that declares the MXFP4 caches).
"""
from __future__ import annotations

import numpy as np

from .formats import decode_bf16_bytes, decode_e4m3, decode_mxfp4_page

BLOCK = 128
PAGE16 = 16


def _k_offsets(esize: int) -> np.ndarray:
    """Byte offset of element (key c, dim d) of a 16-token K page -> [16, 128]."""
    c = np.arange(PAGE16)[:, None]
    d = np.arange(128)[None, :]
    dpc = 16 // esize
    return 1024 * ((d % 32) // dpc) + 256 * (d // 32) + 16 * c + esize * (d % dpc)


def _v_offsets(esize: int) -> np.ndarray:
    """Byte offset of element (key t, dim d) of a 16-token V page -> [16, 128]."""
    t = np.arange(PAGE16)[:, None]
    d = np.arange(128)[None, :]
    dt, c = d // 16, d % 16
    tpc = 4 // esize
    return 1024 * (dt // tpc) + 256 * (t // 4) + 16 * c + 4 * esize * (dt % tpc) + esize * (t % 4)


def _gather_elements(pages: np.ndarray, offsets: np.ndarray, esize: int) -> np.ndarray:
    """pages [n, bytes] -> the raw element bytes in (key, dim) order [n, 16, 128 * esize]."""
    idx = (offsets[..., None] + np.arange(esize)).reshape(PAGE16, 128 * esize)
    return pages[:, idx]


def index_block_keys(idx_pool: np.ndarray, dtype: str, idx_scale: float, block_ids) -> np.ndarray:
    """Index keys of the given blocks -> float64 [n, 128 tok, 128 dim]."""
    pages = np.asarray(idx_pool)[np.asarray(block_ids, dtype=np.int64)]
    n = pages.shape[0]
    if dtype in ("bf16", "fp8"):
        e = 2 if dtype == "bf16" else 1
        tiles = pages.reshape(n * (BLOCK // PAGE16), -1)
        raw = _gather_elements(tiles, _k_offsets(e), e)
        if dtype == "bf16":
            return decode_bf16_bytes(raw).reshape(n, BLOCK, 128)
        return decode_e4m3(raw).reshape(n, BLOCK, 128) * float(idx_scale)
    if dtype == "mxfp4":
        return decode_mxfp4_page(pages)
    raise ValueError(dtype)


def request_index_keys(idx_pool, dtype, idx_scale, block_table_row, length: int) -> np.ndarray:
    """The first ``length`` index keys of one request, in position order -> [length, 128]."""
    nb = -(-length // BLOCK)
    if nb == 0:
        return np.zeros((0, 128))
    keys = index_block_keys(idx_pool, dtype, idx_scale, np.asarray(block_table_row)[:nb])
    return keys.reshape(nb * BLOCK, 128)[:length]


def kv_page_tokens(k_pool, v_pool, dtype: str, page_ids, k_scale: float, v_scale: float,
                   head: int = 0, num_kv_heads: int = 1):
    """Decode whole K/V pages of one KV head -> (K, V), each float64 [n, page tokens, 128].

    ``page_ids`` address both pools: the same id is the K page and the V page."""
    ids = np.asarray(page_ids, dtype=np.int64)
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    kp = k_pool.reshape(k_pool.shape[0], num_kv_heads, -1)[ids, head]
    vp = v_pool.reshape(v_pool.shape[0], num_kv_heads, -1)[ids, head]
    n = ids.shape[0]
    if dtype == "mxfp4":
        return decode_mxfp4_page(kp), decode_mxfp4_page(vp)
    if dtype == "bf16":
        k = decode_bf16_bytes(_gather_elements(kp, _k_offsets(2), 2)).reshape(n, PAGE16, 128)
        v = decode_bf16_bytes(_gather_elements(vp, _v_offsets(2), 2)).reshape(n, PAGE16, 128)
    elif dtype == "fp8":
        k = decode_e4m3(_gather_elements(kp, _k_offsets(1), 1)).reshape(n, PAGE16, 128) * float(k_scale)
        v = decode_e4m3(_gather_elements(vp, _v_offsets(1), 1)).reshape(n, PAGE16, 128) * float(v_scale)
    else:
        raise ValueError(dtype)
    return k, v
