"""The steps of one indexed block-sparse prefill layer, in float64: query tokens
of any requests, in any order, each with its own request and position.

Test infrastructure only (see the package docstring).

Source: the vLLM API page for ``vllm.models.minimax_m3.amd.sparse_attention_msa``,
the prefill branch of ``MiniMaxM3SparseAiterPAImpl.forward``.  The prefill
call takes, beside the query, the caches, the selection and the block table
of the prefill requests, two per-token arrays, ``query_req_id`` and
``query_abs_pos``, and writes the same sparse page table and sparse lengths
as the decode call (rows ``t H_kv + g`` of the table buffer).

Readings where the page is silent:
  * ``query_req_id[t]`` is the row of the block table that holds token t's
    request (the prefill block table is the prefill requests' rows);
  * ``query_abs_pos[t]`` is the token's 0-based position in its request, and
    the token is already in the cache (the writer runs before the attention,
    as in decode, where the lengths count the new tokens), so it attends to
    positions 0 .. abs_pos: causal length L_t = abs_pos + 1 and
    n_t = ceil(L_t / 128) valid blocks;
  * every other rule is the decode layer's (``oracle.decode``): the block score
    over the causally valid keys, the forced tail block n_t - 1, ties to the
    lower block, ascending output padded with -1, the sparse length
    (m - 1) 128 + (L_t - 128 (n_t - 1)).
Token order is free: nothing here depends on tokens of one request being
adjacent or sorted.  The decode layer is the special case where request r's
tokens are the last q positions of a request of length seq_lens[r], in order.
"""
from __future__ import annotations

import numpy as np

from .pools import BLOCK, request_index_keys


def token_lengths(query_abs_pos) -> np.ndarray:
    """Causal length L_t = abs_pos + 1 of every token (int64)."""
    return np.asarray(query_abs_pos, dtype=np.int64) + 1


def _blocks(length) -> int:
    return -(-int(length) // BLOCK)


def _check(query_req_id, query_abs_pos, num_reqs, max_blocks):
    req = np.asarray(query_req_id, dtype=np.int64)
    pos = np.asarray(query_abs_pos, dtype=np.int64)
    assert req.shape == pos.shape and req.ndim == 1
    assert np.all((req >= 0) & (req < num_reqs)), "query_req_id out of range"
    assert np.all((pos >= 0) & (pos < BLOCK * max_blocks)), "query_abs_pos out of range"
    return req, pos


def index_score_prefill(q_idx, idx_pool, idx_dtype, idx_scale, block_table, query_req_id,
                        query_abs_pos, num_kv_heads, max_blocks):
    """Block scores, float64 [H_kv, T, max_blocks]: for token t and KV group g,
    sum over the group's index heads of the largest q_idx[t, h] . k_j over the
    keys j of block b at positions <= abs_pos[t]; -inf for b >= n_t."""
    q_idx = np.asarray(q_idx, dtype=np.float64)
    T, H_idx, _ = q_idx.shape
    req, pos = _check(query_req_id, query_abs_pos, len(block_table), max_blocks)
    assert req.size == T and H_idx % num_kv_heads == 0
    per = H_idx // num_kv_heads
    out = np.full((num_kv_heads, T, max_blocks), -np.inf)
    lens = token_lengths(pos)
    for r in np.unique(req):
        toks = np.flatnonzero(req == r)
        keys = request_index_keys(idx_pool, idx_dtype, idx_scale, block_table[r],
                                  int(lens[toks].max()))                        # [Lmax, 128]
        for t in toks:
            Lt = int(lens[t])
            nt = _blocks(Lt)
            dots = keys[:Lt] @ q_idx[t].T                                        # [Lt, H_idx]
            padded = np.full((nt * BLOCK, H_idx), -np.inf)
            padded[:Lt] = dots
            head_block = padded.reshape(nt, BLOCK, H_idx).max(axis=1)            # [nt, H_idx]
            for g in range(num_kv_heads):
                out[g, t, :nt] = head_block[:, g * per:(g + 1) * per].sum(axis=1)
    return out


def topk_select_prefill(scores, query_abs_pos, top_k):
    """Selections int32 [H_kv, T, top_k]: token t's tail block n_t - 1 plus the
    best top_k - 1 of blocks [0, n_t - 1) by score (ties to the lower block,
    NaN below every number), ascending, padded with -1."""
    scores = np.asarray(scores)
    H_kv, T, _ = scores.shape
    lens = token_lengths(query_abs_pos)
    assert lens.size == T
    out = np.full((H_kv, T, top_k), -1, dtype=np.int32)
    for t in range(T):
        tail = _blocks(lens[t]) - 1
        cand = np.arange(tail)
        for g in range(H_kv):
            s = scores[g, t, :tail]
            nan = np.isnan(s)
            order = np.lexsort((cand, -np.where(nan, 0.0, s), nan))
            sel = np.sort(np.append(cand[order[: min(top_k - 1, tail)]], tail))
            out[g, t, : sel.size] = sel
    return out


def emit_sparse_block_table_prefill(topk, block_table, query_req_id, query_abs_pos, num_kv_heads,
                                    top_k, pages_per_block):
    """Sparse page table int32 [T H_kv, top_k ppb] and sparse lengths int32
    [T H_kv]: selected block b of token t expands into pages
    block_table[req[t]][b] ppb + p, p < ppb; unused slots -1."""
    topk = np.asarray(topk)
    H_kv, T, K = topk.shape
    assert H_kv == num_kv_heads and K == top_k
    req = np.asarray(query_req_id, dtype=np.int64)
    lens = token_lengths(query_abs_pos)
    ppb = int(pages_per_block)
    sbt = np.full((T * H_kv, K * ppb), -1, dtype=np.int32)
    sctx = np.zeros(T * H_kv, dtype=np.int32)
    for t in range(T):
        Lt = int(lens[t])
        nt = _blocks(Lt)
        for g in range(H_kv):
            row = t * H_kv + g
            sel = [int(b) for b in topk[g, t] if b >= 0]
            for k, b in enumerate(sel):
                base = int(block_table[req[t]][b]) * ppb
                sbt[row, k * ppb:(k + 1) * ppb] = base + np.arange(ppb)
            sctx[row] = (len(sel) - 1) * BLOCK + (Lt - BLOCK * (nt - 1))
    return sbt, sctx


def prefill_layer(q, q_idx, idx_pool, idx_dtype, idx_scale, k_pool, v_pool, kv_dtype, k_scale,
                  v_scale, block_table, query_req_id, query_abs_pos, num_kv_heads, max_blocks, top_k,
                  pages_per_block, sm_scale):
    """Score -> select -> emit -> attend for a ragged batch of prefill tokens.

    The attention is the decode layer's (``oracle.decode.sparse_pa_decode``):
    it reads only the sparse page table and lengths, whatever token they
    belong to."""
    from .decode import sparse_pa_decode

    scores = index_score_prefill(q_idx, idx_pool, idx_dtype, idx_scale, block_table, query_req_id,
                                 query_abs_pos, num_kv_heads, max_blocks)
    topk = topk_select_prefill(scores, query_abs_pos, top_k)
    sbt, sctx = emit_sparse_block_table_prefill(topk, block_table, query_req_id, query_abs_pos,
                                                num_kv_heads, top_k, pages_per_block)
    out = sparse_pa_decode(q, k_pool, v_pool, kv_dtype, k_scale, v_scale, sbt, sctx, num_kv_heads,
                           pages_per_block, sm_scale)
    return {"scores": scores, "topk": topk, "sparse_bt": sbt, "sparse_ctx": sctx, "out": out}
