"""Helpers shared by the GPU parity tests: host copies for the oracle, the
tolerances, and per-request sampling of full-size workloads."""
from __future__ import annotations

from dataclasses import replace

import numpy as np
import torch

from indexer_selected_block_amd import workload as wl
from oracle import decode as od
from oracle import formats, pools

# Tolerances: scores within 1e-3 relative; attention within
# 1e-2 max|V| + 1e-3 (fp8 / MXFP4 K/V) or 4e-3 max|V| (bf16 K/V).
SCORE_RTOL = 1e-3


def attn_tol(kv_dtype: str, vmax: float) -> float:
    return 4e-3 * vmax if kv_dtype == "bf16" else 1e-2 * vmax + 1e-3


def small_configs():
    c = wl.CONFIGS
    return {
        "tiny_bf16": c["tiny_bf16"],
        "fp8_decode": wl.shrink(c["fp8_decode"], num_reqs=5, ctx_lo=700, ctx_hi=5000),
        "spec_decode": wl.shrink(c["spec_decode"], num_reqs=6, ctx_lo=300, ctx_hi=3000, num_pad_reqs=2),
        "mxfp4": wl.shrink(c["mxfp4"], num_reqs=3, ctx_lo=900, ctx_hi=3000),
        "long_context": wl.shrink(c["long_context"], num_reqs=2, ctx_lo=5000, ctx_hi=9000),
        # prefill chunks (more than 16 tokens or 64 index rows: the wide scorer),
        # each with a ragged last query tile, for every index key type
        "prefill": replace(wl.shrink(c["prefill"], num_reqs=2, ctx_lo=600, ctx_hi=3000), query_len=150),
        "prefill_mxfp4": replace(wl.shrink(c["mxfp4"], num_reqs=2, ctx_lo=900, ctx_hi=2500), query_len=37),
        "prefill_bf16": replace(c["tiny_bf16"], name="prefill_bf16", query_len=70, ctx_lo=700, ctx_hi=1024),
    }


def host_inputs(w):
    """Numpy views of a workload on the CPU, decoded queries included."""
    h = w.to("cpu")
    cfg = h.cfg
    return dict(
        cfg=cfg, seq_lens=h.seq_lens.numpy(), block_table=h.block_table.numpy(),
        q=formats.decode_query(h.q.numpy(), cfg.q_dtype),
        q_idx=formats.decode_query(h.q_idx.numpy(), cfg.qidx_dtype),
        idx_pool=h.idx_pool.numpy(), k_pool=h.k_pool.numpy(), v_pool=h.v_pool.numpy(),
        idx_scale=h.idx_scale, k_scale=h.k_scale, v_scale=h.v_scale, sm_scale=h.sm_scale)


def oracle_scores(hi):
    cfg = hi["cfg"]
    return od.index_score(hi["q_idx"], hi["idx_pool"], cfg.idx_dtype, hi["idx_scale"],
                          hi["block_table"], hi["seq_lens"], cfg.query_len, cfg.num_kv_heads,
                          cfg.max_blocks)


def assert_scores_close(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape
    assert not np.isnan(ref).any() and not np.isnan(gpu).any(), "NaN score (poison read?)"
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), "-inf pattern differs"
    fin = np.isfinite(ref)
    rowmax = np.where(fin, np.abs(ref), 0).max(axis=-1, keepdims=True)
    scale = np.maximum(np.abs(ref), 1e-3 * rowmax)
    with np.errstate(invalid="ignore"):
        err = np.abs(gpu - ref)
    bad = fin & (err > SCORE_RTOL * scale)
    assert not bad.any(), f"{bad.sum()} scores out of tolerance; worst {np.max(err[fin] / scale[fin]):.3g}"


def attended_vmax(hi, sparse_bt, sparse_ctx):
    """max |V| over the dequantised V of the positions the rows attend."""
    cfg = hi["cfg"]
    ptok = 128 // cfg.pages_per_block
    best = 0.0
    for row in range(sparse_bt.shape[0]):
        n = int(sparse_ctx[row])
        if n == 0:
            continue
        npg = -(-n // ptok)
        _, V = pools.kv_page_tokens(hi["k_pool"], hi["v_pool"], cfg.kv_dtype, sparse_bt[row, :npg],
                                    hi["k_scale"], hi["v_scale"], head=row % cfg.num_kv_heads,
                                    num_kv_heads=cfg.num_kv_heads)
        best = max(best, float(np.abs(V.reshape(-1, 128)[:n]).max()))
    return best


def oracle_attention(hi, sparse_bt, sparse_ctx):
    cfg = hi["cfg"]
    return od.sparse_pa_decode(hi["q"], hi["k_pool"], hi["v_pool"], cfg.kv_dtype, hi["k_scale"],
                               hi["v_scale"], sparse_bt, sparse_ctx, cfg.num_kv_heads,
                               cfg.pages_per_block, hi["sm_scale"])


def selection_margin_ok(ref_scores_row, nt, K, gpu_sel, tol):
    """Is the GPU selection a valid top-k for fp64 scores known to within `tol`?

    The tail must be present; every chosen candidate must score at least the
    (K-1)-th best minus tol, and every rejected one at most it plus tol."""
    tail = nt - 1
    sel = [b for b in gpu_sel if b >= 0]
    if nt == 0:
        return len(sel) == 0
    if tail not in sel or len(sel) != min(K, nt):
        return False
    if K >= nt:
        return sel == list(range(nt))
    cand = ref_scores_row[:tail]
    kth = np.sort(cand)[::-1][K - 2] if K > 1 else np.inf
    chosen = [b for b in sel if b != tail]
    rejected = [b for b in range(tail) if b not in chosen]
    return all(cand[b] >= kth - tol for b in chosen) and all(cand[b] <= kth + tol for b in rejected)


# ---------------------------------------------------------------- sampling
def sample_requests(w, reqs):
    """Host inputs for a subset of requests of a (large) device workload.

    Only the blocks those requests use are copied; they are renumbered 0..n-1
    (plus a poison block) in a compact pool.  Returns (host inputs, the
    requests' query tokens, the map from device block id to compact block id)."""
    cfg = w.cfg
    reqs = list(reqs)
    lens = w.seq_lens[reqs].cpu().numpy()
    bt = w.block_table[reqs].cpu().numpy()
    nblk = [(-(-int(L) // 128)) for L in lens]
    used = np.concatenate([bt[i, :n] for i, n in enumerate(nblk)] + [np.zeros(0, dtype=np.int32)])
    poison = cfg.pool_blocks
    ids = np.concatenate([used, [poison]]).astype(np.int64)
    remap = {int(b): i for i, b in enumerate(ids)}
    bt_c = np.full_like(bt, len(ids) - 1)
    for i, n in enumerate(nblk):
        bt_c[i, :n] = [remap[int(b)] for b in bt[i, :n]]
    sel = torch.from_numpy(ids).to(w.idx_pool.device)
    ppb = cfg.pages_per_block
    kv_blocks = lambda pool: pool.view(pool.shape[0] // ppb, -1)  # noqa: E731
    idx_pool = w.idx_pool[sel].cpu().numpy()
    k_pool = kv_blocks(w.k_pool)[sel].cpu().reshape(len(ids) * ppb, -1).numpy()
    v_pool = kv_blocks(w.v_pool)[sel].cpu().reshape(len(ids) * ppb, -1).numpy()
    ql = cfg.query_len
    toks = [r * ql + i for r in reqs for i in range(ql)]
    tsel = torch.tensor(toks, device=w.q.device)
    sub = wl.replace(cfg, num_reqs=len(reqs), num_pad_reqs=0, pool_blocks=len(ids) - 1)
    hi = dict(
        cfg=sub, seq_lens=lens, block_table=bt_c,
        q=formats.decode_query(w.q[tsel].cpu().numpy(), cfg.q_dtype),
        q_idx=formats.decode_query(w.q_idx[tsel].cpu().numpy(), cfg.qidx_dtype),
        idx_pool=idx_pool, k_pool=k_pool, v_pool=v_pool, idx_scale=w.idx_scale,
        k_scale=w.k_scale, v_scale=w.v_scale, sm_scale=w.sm_scale)
    return hi, toks, remap


def compact_pages(sparse_bt, remap, ppb):
    """Device page ids of a sparse table -> the compact pool's (page = block
    ppb + slot); -1 stays -1."""
    out = np.full_like(sparse_bt, -1)
    for idx, pg in np.ndenumerate(sparse_bt):
        if pg >= 0:
            out[idx] = remap[int(pg) // ppb] * ppb + int(pg) % ppb
    return out


def check_chain(hi, scores_gpu, topk_gpu, sbt_gpu, sctx_gpu, out_gpu, ref, bt_global, remap=None):
    """A GPU layer step by step against the oracle fed the GPU's own results
    (every row, no exemptions):

    * scores: the GPU's fp32 scores against the oracle's fp64 scores, within
      the score tolerance, the -inf set exact;
    * selection: the oracle's top-k run on the GPU's own fp32 scores must equal
      the GPU's selection bit for bit;
    * table: the oracle's emit of that selection must equal the GPU's table and
      lengths bit for bit;
    * output: the oracle's attention over the GPU's own table must match the
      GPU's output on every row within the attention tolerance.

    Besides, the GPU's selection must be a valid top-k of the oracle's fp64
    scores to within the GPU's score error on every row (rows may pick a
    different member of a near-tie, never a clearly worse block).
    ``remap`` maps device block ids to the compact pool of sampled requests."""
    cfg = hi["cfg"]
    ql, H_kv, K, ppb = cfg.query_len, cfg.num_kv_heads, cfg.top_k, cfg.pages_per_block
    T = len(hi["seq_lens"]) * ql
    scores32 = np.asarray(scores_gpu, dtype=np.float32)
    assert_scores_close(scores32, ref["scores"])
    # selection: the oracle on the GPU's own fp32 scores, bit-exact
    topk_ref = od.topk_select(scores32, hi["seq_lens"], ql, K)
    diff = np.nonzero(~np.all(topk_ref == topk_gpu, axis=-1))
    assert diff[0].size == 0, f"{diff[0].size} rows select differently from the oracle on the same " \
                              f"scores; first (g, t) = {(int(diff[0][0]), int(diff[1][0]))}"
    # and a valid top-k of the fp64 scores within the GPU's score error
    with np.errstate(invalid="ignore"):
        err_row = np.where(np.isfinite(ref["scores"]), np.abs(scores32 - ref["scores"]), 0).max(axis=-1)
    for g in range(H_kv):
        for t in range(T):
            if np.array_equal(topk_gpu[g, t], ref["topk"][g, t]):
                continue
            r, i = divmod(t, ql)
            nt = od.num_blocks(od.causal_length(hi["seq_lens"][r], ql, i))
            assert selection_margin_ok(ref["scores"][g, t], nt, K, list(topk_gpu[g, t]), 2 * err_row[g, t] + 1e-12), \
                f"row ({g},{t}): GPU selection is not a top-{K} of the oracle scores"
    # table: the oracle's emit of the GPU's selection, bit-exact
    sbt_ref, sctx_ref = od.emit_sparse_block_table(topk_gpu, bt_global, hi["seq_lens"], ql, H_kv, K, ppb)
    assert np.array_equal(sbt_gpu, sbt_ref), "sparse page table differs"
    assert np.array_equal(sctx_gpu, sctx_ref), "sparse lengths differ"
    # output: the oracle's attention over the GPU's own table, every row
    sbt_host = sbt_gpu if remap is None else compact_pages(sbt_gpu, remap, ppb)
    out_ref = oracle_attention(hi, sbt_host, sctx_gpu)
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hi, sbt_host, sctx_gpu))
    assert np.isfinite(out_gpu).all(), "NaN in the attention output"
    err = np.abs(out_gpu - out_ref).max(axis=(1, 2))
    assert (err <= tol).all(), f"attention err {err.max():.4g} > {tol:.4g} on {(err > tol).sum()} tokens"


def oracle_layer(hi):
    cfg = hi["cfg"]
    return od.decode_layer(hi["q"], hi["q_idx"], hi["idx_pool"], cfg.idx_dtype, hi["idx_scale"],
                           hi["k_pool"], hi["v_pool"], cfg.kv_dtype, hi["k_scale"], hi["v_scale"],
                           hi["block_table"], hi["seq_lens"], cfg.query_len, cfg.num_kv_heads,
                           cfg.max_blocks, cfg.top_k, cfg.pages_per_block, hi["sm_scale"])


def shard_candidates(scores, lens, G, K, rng):
    """Candidates of each decode row (q = 1) from G contiguous shards of its
    blocks, each selected by topk_select as a whole row: ids [H, T, G K] with
    their scores, -1 padded, shuffled."""
    H, T, MB = scores.shape
    ids = np.full((H, T, G * K), -1, dtype=np.int32)
    sc = np.zeros((H, T, G * K), dtype=scores.dtype)
    for t in range(T):
        n = min(od.num_blocks(int(lens[t])), MB)
        if n == 0:
            continue
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(G, n) - 1, replace=False)) if n > 1 else []
        bounds = np.concatenate([[0], cuts, [n]]).astype(int)
        for g in range(H):
            picks = []
            for a, b in zip(bounds[:-1], bounds[1:]):
                sel = od.topk_select(scores[g:g + 1, t:t + 1, a:b], np.array([(b - a) * 128]), 1, K)[0, 0]
                picks += [a + int(x) for x in sel if x >= 0]
            picks = rng.permutation(picks)
            ids[g, t, :len(picks)] = picks
            sc[g, t, :len(picks)] = scores[g, t, picks]
    return sc, ids

