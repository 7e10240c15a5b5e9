"""The four steps of one indexed block-sparse paged-attention decode layer, in float64.

Test infrastructure only (see the package docstring).

Notation: R requests, q = decode_query_len, T = R q query tokens; token
t = r q + i (i < q) of request r has causal length
L_t = max(0, seq_lens[r] - (q - 1 - i)) and n_t = ceil(L_t / 128) valid
128-token blocks.  H_kv KV heads, H_q query heads (G = H_q / H_kv per KV head),
H_idx index heads (H_idx / H_kv per KV head), head dim 128.

Sources: ROCm/ATOM PR 2962 ("[MiniMax-M3.1] MXFP4 index cache and MXFP4 KV
cache") and the vLLM API page for ``vllm.models.minimax_m3.amd.sparse_attention_msa``
(the decode call of ``MiniMaxM3SparseAiterPAImpl.forward``).
"""
from __future__ import annotations

import numpy as np

from .pools import BLOCK, kv_page_tokens, request_index_keys


def causal_length(seq_len: int, q_len: int, i: int) -> int:
    """L_t for query token i of a request of length seq_len.

    Floored at 0, so the rows of a pad request (length 0) with q > 1 select
    and attend nothing (PR 2962, the pad-row fix: the emit step floors a row's
    causal length at zero on entry)."""
    return max(0, int(seq_len) - (q_len - 1 - i))


def num_blocks(length: int) -> int:
    return -(-int(length) // BLOCK)


def index_score(q_idx, idx_pool, idx_dtype, idx_scale, block_table, seq_lens, q_len,
                num_kv_heads, max_blocks):
    """Block scores, float64 [H_kv, T, max_blocks].

    The sources fix that the scorer yields one fp32 score per (index head, row,
    128-token block) (PR 2962, Known limits: the H x rows x blocks x 4 B
    workspace) and that the index query is e4m3 for the MXFP4 index (Summary).
    Readings where they are silent:
      * a head's block score is the largest dot product q_idx[t,h] . k_j over the
        block's causally valid tokens j (position < L_t);
      * the index heads of one KV group are summed into that group's score, the
        selection being made per (token, KV head);
      * no scale factor other than the fp8 index cache's per-tensor scale;
      * blocks b >= n_t score -inf.
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    T, H_idx, _ = q_idx.shape
    R = len(seq_lens)
    assert T == R * q_len and H_idx % num_kv_heads == 0
    per = H_idx // num_kv_heads
    out = np.full((num_kv_heads, T, max_blocks), -np.inf)
    for r in range(R):
        L = int(seq_lens[r])
        if L == 0:
            continue
        keys = request_index_keys(idx_pool, idx_dtype, idx_scale, block_table[r], L)   # [L, 128]
        for i in range(q_len):
            t = r * q_len + i
            Lt = causal_length(L, q_len, i)
            nt = num_blocks(Lt)
            if nt == 0:
                continue
            dots = keys[:Lt] @ q_idx[t].T                                        # [Lt, H_idx]
            padded = np.full((nt * BLOCK, H_idx), -np.inf)
            padded[:Lt] = dots
            head_block = padded.reshape(nt, BLOCK, H_idx).max(axis=1)            # [nt, H_idx]
            for g in range(num_kv_heads):
                out[g, t, :nt] = head_block[:, g * per:(g + 1) * per].sum(axis=1)
    return out


def topk_select(scores, seq_lens, q_len, top_k):
    """Selected block indices, int32 [H_kv, T, top_k], ascending, padded with -1.

    Per row: the tail block n_t - 1 is part of every selection (PR 2962, the
    decode commit keeps the tail page; ``sparse_local_block`` is checked at
    startup); the other top_k - 1 are the best of blocks [0, n_t - 1) by
    score, ties to the lower block index.  A row with n_t = 0 selects nothing
    (Pad-row fix).  Readings: NaN ranks below every number, -0.0 equals +0.0,
    the output is ascending by block index (so the tail is last) and unused
    slots are -1.  Scores are compared in the precision they are given in.
    """
    scores = np.asarray(scores)
    H_kv, T, _ = scores.shape
    out = np.full((H_kv, T, top_k), -1, dtype=np.int32)
    for t in range(T):
        r, i = divmod(t, q_len)
        nt = num_blocks(causal_length(seq_lens[r], q_len, i))
        if nt == 0:
            continue
        tail = nt - 1
        cand = np.arange(tail)
        for g in range(H_kv):
            s = scores[g, t, :tail]
            nan = np.isnan(s)
            key = np.where(nan, 0.0, s)
            # lexsort: last key is primary -> non-NaN first, then score descending,
            # then block index ascending.
            order = np.lexsort((cand, -key, nan))
            chosen = cand[order[: min(top_k - 1, tail)]]
            sel = np.sort(np.append(chosen, tail))
            out[g, t, : sel.size] = sel
    return out


def merge_candidates(cand_scores, cand_ids, seq_lens, q_len, top_k, max_blocks):
    """Selections [H_kv, T, top_k] from per-row candidates: cand_ids [H_kv, T, C]
    block ids (distinct in a row; -1 = empty) with their scores.

    The merge step of context parallelism (PR 2962 names the candidate exchange
    among the users of the emit helper; the reading: shards of a row's blocks
    each select as if they were the whole row, and the union of their picks,
    with scores, is merged).  Per row: the tail block n_t - 1 plus the best
    top_k - 1 candidates with ids in [0, n_t - 1), in topk_select's order; a
    row with n_t - 1 <= top_k - 1 takes all its blocks, as topk_select does.
    """
    cs = np.asarray(cand_scores)
    ci = np.asarray(cand_ids)
    H_kv, T, _ = ci.shape
    out = np.full((H_kv, T, top_k), -1, dtype=np.int32)
    for t in range(T):
        r, i = divmod(t, q_len)
        nt = min(num_blocks(causal_length(seq_lens[r], q_len, i)), max_blocks)
        if nt == 0:
            continue
        tail = nt - 1
        for g in range(H_kv):
            if tail <= top_k - 1:
                sel = np.arange(nt)
            else:
                ok = (ci[g, t] >= 0) & (ci[g, t] < tail)
                ids, sc = ci[g, t][ok], cs[g, t][ok]
                nan = np.isnan(sc)
                order = np.lexsort((ids, -np.where(nan, 0.0, sc), nan))
                sel = np.sort(np.append(ids[order[: top_k - 1]], tail))
            out[g, t, : sel.size] = sel
    return out


def emit_sparse_block_table(topk, block_table, seq_lens, q_len, num_kv_heads, top_k,
                            pages_per_block):
    """Sparse page table int32 [T H_kv, top_k ppb] and sparse lengths int32 [T H_kv].

    Row (t, g) is row t H_kv + g, token-major (vLLM API page, ``forward``: the
    ``sparse_bt_buffer[: nd * kvh]`` slice); the selection is head-major
    ``[H_kv, T, K]`` (``topk[:, :nd, :]``).  A selected block b expands into
    pages ``block_table[r][b] ppb + p`` for p < ppb (PR 2962: pages_per_block 8
    for the page-16 cache, 1 for page-128 caches).  The sparse length counts
    128 tokens for every selected block but the tail, plus the tail's
    L_t - 128 (n_t - 1) tokens; rows with n_t = 0 are empty.  Reading: unused
    slots are -1.
    """
    topk = np.asarray(topk)
    H_kv, T, K = topk.shape
    assert H_kv == num_kv_heads and K == top_k
    ppb = int(pages_per_block)
    sbt = np.full((T * H_kv, K * ppb), -1, dtype=np.int32)
    sctx = np.zeros(T * H_kv, dtype=np.int32)
    for t in range(T):
        r, i = divmod(t, q_len)
        Lt = causal_length(seq_lens[r], q_len, i)
        nt = num_blocks(Lt)
        for g in range(H_kv):
            row = t * H_kv + g
            sel = [int(b) for b in topk[g, t] if b >= 0]
            if nt == 0 or not sel:
                continue
            for k, b in enumerate(sel):
                base = int(block_table[r][b]) * ppb
                for p in range(ppb):
                    sbt[row, k * ppb + p] = base + p
            sctx[row] = (len(sel) - 1) * BLOCK + (Lt - BLOCK * (nt - 1))
    return sbt, sctx


def sparse_pa_decode(q, k_pool, v_pool, kv_dtype, k_scale, v_scale, sparse_bt, sparse_ctx,
                     num_kv_heads, pages_per_block, sm_scale):
    """Attention over the sparse positions, float64 [T, H_q, 128].

    The decode call of the vLLM API page (``minimax_m3_sparse_attn_decode_aiter``
    with the emitted ``sparse_block_table`` / ``sparse_context_lens``): for row
    (t, g) and query head h of group g, z_u = scale q[t,h] . K_u over sparse
    positions u < sparse_ctx, softmax over u, output sum_u p_u V_u.  Position u
    is slot u mod P of page sparse_bt[row][u div P], P = 128 / ppb tokens a page.
    Row (t, g) reads KV head g's page under each page id.  Readings: a row of
    length 0 outputs zeros; fp8 K/V carry per-tensor scales.
    """
    q = np.asarray(q, dtype=np.float64)
    T, H_q, D = q.shape
    G = H_q // num_kv_heads
    ptok = BLOCK // int(pages_per_block)
    out = np.zeros((T, H_q, D))
    for t in range(T):
        for g in range(num_kv_heads):
            row = t * num_kv_heads + g
            n = int(sparse_ctx[row])
            if n == 0:
                continue
            npages = -(-n // ptok)
            K, V = kv_page_tokens(k_pool, v_pool, kv_dtype, sparse_bt[row, :npages], k_scale, v_scale,
                                  head=g, num_kv_heads=num_kv_heads)
            K = K.reshape(npages * ptok, D)[:n]
            V = V.reshape(npages * ptok, D)[:n]
            qh = q[t, g * G:(g + 1) * G]
            z = sm_scale * (qh @ K.T)                                   # [G, n]
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            out[t, g * G:(g + 1) * G] = (p @ V) / p.sum(axis=1, keepdims=True)
    return out


def decode_layer(q, q_idx, idx_pool, idx_dtype, idx_scale, k_pool, v_pool, kv_dtype, k_scale,
                 v_scale, block_table, seq_lens, q_len, num_kv_heads, max_blocks, top_k,
                 pages_per_block, sm_scale):
    """Score -> select -> emit -> attend, each step fed the previous step's float64 result."""
    scores = index_score(q_idx, idx_pool, idx_dtype, idx_scale, block_table, seq_lens, q_len,
                         num_kv_heads, max_blocks)
    topk = topk_select(scores, seq_lens, q_len, top_k)
    sbt, sctx = emit_sparse_block_table(topk, block_table, seq_lens, q_len, num_kv_heads, top_k,
                                        pages_per_block)
    out = sparse_pa_decode(q, k_pool, v_pool, kv_dtype, k_scale, v_scale, sbt, sctx,
                           num_kv_heads, pages_per_block, sm_scale)
    return {"scores": scores, "topk": topk, "sparse_bt": sbt, "sparse_ctx": sctx, "out": out}
