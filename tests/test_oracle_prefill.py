"""Pins for the oracle's ragged prefill steps (CPU only).

Each is checked against something other than its own code: the decode
oracle (pinned by its own tests) on the uniform-chunk special case, torch's
scaled_dot_product_attention when every block is selected (dense causal
attention per token, each at its own position), pure-Python brute force on
tiny inputs, and invariants the per-token form implies (token order is free;
a token sees nothing past its own position).
"""
import math

import numpy as np
import pytest
import torch

from indexer_selected_block_amd import workload as wl
from oracle import decode as od
from oracle import formats
from oracle import prefill as op

import _pages


def _decoded(w, batch):
    cfg = w.cfg
    q = formats.decode_query(batch.q.numpy(), cfg.q_dtype)
    q_idx = formats.decode_query(batch.q_idx.numpy(), cfg.qidx_dtype)
    return q, q_idx


def _layer(w, batch, top_k=None, req=None, pos=None, q=None, q_idx=None, k_pool=None, v_pool=None,
           idx_pool=None):
    cfg = w.cfg
    dq, dqi = _decoded(w, batch)
    return op.prefill_layer(
        dq if q is None else q, dqi if q_idx is None else q_idx,
        (w.idx_pool.numpy() if idx_pool is None else idx_pool), cfg.idx_dtype, w.idx_scale,
        (w.k_pool.numpy() if k_pool is None else k_pool), (w.v_pool.numpy() if v_pool is None else v_pool),
        cfg.kv_dtype, w.k_scale, w.v_scale, w.block_table.numpy(),
        batch.query_req_id.numpy() if req is None else req,
        batch.query_abs_pos.numpy() if pos is None else pos,
        cfg.num_kv_heads, cfg.max_blocks, cfg.top_k if top_k is None else top_k, cfg.pages_per_block,
        w.sm_scale)


def _small(name="prefill_ragged", num_reqs=5, lo=200, hi=900, **kw):
    base = wl.ragged_config(name) if name in wl.RAGGED_CHUNKS else wl.CONFIGS[name]
    return wl.make_workload(wl.shrink(base, num_reqs=num_reqs, ctx_lo=lo, ctx_hi=hi, num_pad_reqs=0, **kw))


# ---------------------------------------------------------------- reduction to decode
@pytest.mark.parametrize("name", ["spec_decode", "mxfp4"])
def test_uniform_chunks_reduce_to_the_decode_layer(name):
    """Request r's tokens at its last q positions, in order: the decode layer's
    batch.  Every output equals the decode oracle's, bit for bit."""
    w = _small(name, num_reqs=3, lo=130, hi=700)
    cfg = w.cfg
    lens = w.seq_lens.numpy()
    q_len = cfg.query_len
    req = np.repeat(np.arange(3), q_len)
    pos = np.concatenate([np.arange(L - q_len, L) for L in lens])
    q = formats.decode_query(w.q.numpy(), cfg.q_dtype)
    q_idx = formats.decode_query(w.q_idx.numpy(), cfg.qidx_dtype)
    dec = od.decode_layer(q, q_idx, w.idx_pool.numpy(), cfg.idx_dtype, w.idx_scale, w.k_pool.numpy(),
                          w.v_pool.numpy(), cfg.kv_dtype, w.k_scale, w.v_scale, w.block_table.numpy(), lens,
                          q_len, cfg.num_kv_heads, cfg.max_blocks, cfg.top_k, cfg.pages_per_block,
                          w.sm_scale)
    pre = op.prefill_layer(q, q_idx, w.idx_pool.numpy(), cfg.idx_dtype, w.idx_scale, w.k_pool.numpy(),
                           w.v_pool.numpy(), cfg.kv_dtype, w.k_scale, w.v_scale, w.block_table.numpy(), req,
                           pos, cfg.num_kv_heads, cfg.max_blocks, cfg.top_k, cfg.pages_per_block, w.sm_scale)
    for key in ("scores", "topk", "sparse_bt", "sparse_ctx", "out"):
        np.testing.assert_array_equal(pre[key], dec[key], err_msg=key)


# ---------------------------------------------------------------- invariants
def test_token_order_is_free():
    """Shuffling the tokens (with their ids and positions) shuffles every output
    the same way and changes nothing else."""
    w = _small()
    chunks = (40, 1, 0, 25, 9)
    b = wl.ragged_batch(w, chunks)
    ref = _layer(w, b)
    perm = np.random.default_rng(3).permutation(b.num_tokens)
    q, q_idx = _decoded(w, b)
    res = _layer(w, b, req=b.query_req_id.numpy()[perm], pos=b.query_abs_pos.numpy()[perm], q=q[perm],
                 q_idx=q_idx[perm])
    np.testing.assert_array_equal(res["scores"], ref["scores"][:, perm])
    np.testing.assert_array_equal(res["topk"], ref["topk"][:, perm])
    H = w.cfg.num_kv_heads
    rows = (perm[:, None] * H + np.arange(H)).reshape(-1)
    np.testing.assert_array_equal(res["sparse_bt"], ref["sparse_bt"][rows])
    np.testing.assert_array_equal(res["sparse_ctx"], ref["sparse_ctx"][rows])
    np.testing.assert_array_equal(res["out"], ref["out"][perm])


def _poison_after(w, r, p):
    """Copies of the pools with every position past p of request r set to NaN
    (index keys, K and V)."""
    cfg = w.cfg
    idx, kp, vp = w.idx_pool.numpy().copy(), w.k_pool.numpy().copy(), w.v_pool.numpy().copy()
    L = int(w.seq_lens[r])
    bt = w.block_table.numpy()[r]
    ppb = cfg.pages_per_block
    assert cfg.idx_dtype == "fp8" and cfg.kv_dtype == "fp8"
    for b in range((p + 1) // 128, -(-L // 128)):
        lo = max(0, p + 1 - 128 * b)
        # index page: eight 16-token tiles in K-page order
        tiles = _pages.read_back(idx[bt[b]].reshape(8, -1), 1, "k")         # [8, 16, 128]
        flat = tiles.reshape(128, 128)
        flat[lo:] = 0x7F
        idx[bt[b]] = _pages.k_pages(flat.reshape(8, 16, 128, 1)).reshape(-1)
        for s in range(lo, 128):
            page = bt[b] * ppb + s // 16
            for pool, kind in ((kp, "k"), (vp, "v")):
                pg = _pages.read_back(pool[page].reshape(1, -1), 1, kind)   # [1, 16, 128]
                pg[0, s % 16] = 0x7F
                builder = _pages.k_pages if kind == "k" else _pages.v_pages
                pool[page] = builder(pg.reshape(1, 16, 128, 1)).reshape(-1)
    return idx, kp, vp


def test_a_token_sees_nothing_past_its_position():
    """A token's scores, selection, table and output are the same when every
    position after its own is NaN, and the same alone as in the batch."""
    w = _small(num_reqs=3, lo=300, hi=600)
    b = wl.ragged_batch(w, (30, 12, 20))
    ref = _layer(w, b)
    q, q_idx = _decoded(w, b)
    for t in (0, 17, 29, 30, 45, b.num_tokens - 1):
        r, p = int(b.query_req_id[t]), int(b.query_abs_pos[t])
        idx, kp, vp = _poison_after(w, r, p)
        one = _layer(w, b, req=np.array([r]), pos=np.array([p]), q=q[t:t + 1], q_idx=q_idx[t:t + 1],
                     k_pool=kp, v_pool=vp, idx_pool=idx)
        np.testing.assert_array_equal(one["scores"][:, 0], ref["scores"][:, t])
        np.testing.assert_array_equal(one["topk"][:, 0], ref["topk"][:, t])
        np.testing.assert_array_equal(one["sparse_ctx"], ref["sparse_ctx"][t:t + 1])
        np.testing.assert_array_equal(one["out"][0], ref["out"][t])
        assert np.isfinite(one["out"]).all()


# ---------------------------------------------------------------- library routine
def test_every_block_selected_is_dense_causal_attention_per_token():
    """top_k >= n_t everywhere: each token's output is torch SDPA over its
    request's positions 0 .. abs_pos (float64, K/V read back by torch's views)."""
    w = _small(num_reqs=4, lo=100, hi=900)
    b = wl.ragged_batch(w, (33, 1, 70, 5), order="shuffled", seed=2)
    res = _layer(w, b, top_k=w.cfg.max_blocks)
    q = torch.from_numpy(formats.decode_query(b.q.numpy(), w.cfg.q_dtype))
    kb = _pages.read_back(w.k_pool.numpy(), 1, "k")
    vb = _pages.read_back(w.v_pool.numpy(), 1, "v")
    view = torch.float8_e4m3fn
    kpages = torch.from_numpy(kb.reshape(kb.shape[0], -1).copy()).view(view).double().reshape(-1, 16, 128)
    vpages = torch.from_numpy(vb.reshape(vb.shape[0], -1).copy()).view(view).double().reshape(-1, 16, 128)
    kpages, vpages = kpages * w.k_scale, vpages * w.v_scale
    Hq = w.cfg.num_q_heads
    for t in range(b.num_tokens):
        r, L = int(b.query_req_id[t]), int(b.query_abs_pos[t]) + 1
        pos = torch.arange(L)
        page = w.block_table[r, pos // 128].long() * 8 + (pos % 128) // 16
        K, V = kpages[page, pos % 16], vpages[page, pos % 16]
        o = torch.nn.functional.scaled_dot_product_attention(
            q[t].reshape(1, Hq, 1, 128), K.expand(1, Hq, L, 128), V.expand(1, Hq, L, 128), scale=w.sm_scale)
        np.testing.assert_allclose(res["out"][t], o.reshape(Hq, 128).numpy(), rtol=1e-10, atol=1e-12)
    assert (res["sparse_ctx"] == b.query_abs_pos.numpy() + 1).all()


# ---------------------------------------------------------------- brute force
def test_scores_topk_and_emit_brute_force_tiny():
    """Pure-Python loops over tokens, blocks, keys and dims on a tiny ragged
    batch with two index heads per KV head and two KV heads."""
    rng = np.random.default_rng(5)
    nblk = 7
    keys = rng.integers(-3, 4, size=(nblk, 128, 128)).astype(np.float64)   # exact in bf16
    kb = torch.from_numpy(keys.astype(np.float32)).to(torch.bfloat16)
    raw = kb.contiguous().view(torch.uint8).numpy().reshape(nblk * 8, 16, 128, 2)
    idx_pool = _pages.k_pages(raw).reshape(nblk, -1)
    bt = np.array([[3, 0, 6], [5, 1, 2]])
    req = np.array([1, 0, 1, 0, 1])
    pos = np.array([300, 0, 129, 200, 127])
    H_idx, H_kv, MB, K = 4, 2, 3, 2
    q_idx = rng.integers(-2, 3, size=(5, H_idx, 128)).astype(np.float64)
    scores = op.index_score_prefill(q_idx, idx_pool, "bf16", 1.0, bt, req, pos, H_kv, MB)
    per = H_idx // H_kv
    for t in range(5):
        L = pos[t] + 1
        for g in range(H_kv):
            for b in range(MB):
                if 128 * b >= L:
                    assert scores[g, t, b] == -math.inf
                    continue
                total = 0.0
                for h in range(g * per, (g + 1) * per):
                    best = -math.inf
                    for j in range(128 * b, min(128 * b + 128, L)):
                        k = keys[bt[req[t]][b]][j - 128 * b]
                        best = max(best, sum(float(q_idx[t, h, d]) * float(k[d]) for d in range(128)))
                    total += best
                assert scores[g, t, b] == total
    topk = op.topk_select_prefill(scores, pos, K)
    sbt, sctx = op.emit_sparse_block_table_prefill(topk, bt, req, pos, H_kv, K, 8)
    for t in range(5):
        L = pos[t] + 1
        nt = -(-L // 128)
        for g in range(H_kv):
            s = scores[g, t]
            best = sorted(range(nt - 1), key=lambda b: (-s[b], b))[: K - 1]
            want = sorted(best + [nt - 1])
            assert list(topk[g, t][: len(want)]) == want and all(topk[g, t][len(want):] == -1)
            row = t * H_kv + g
            pages = [bt[req[t]][b] * 8 + p for b in want for p in range(8)]
            assert list(sbt[row][: len(pages)]) == pages and all(sbt[row][len(pages):] == -1)
            assert sctx[row] == (len(want) - 1) * 128 + L - 128 * (nt - 1)


def test_single_token_at_position_zero():
    """A token at position 0 attends to its own key alone: output V_0, one
    block, sparse length 1."""
    w = _small(num_reqs=2, lo=200, hi=300)
    b = wl.ragged_batch(w, (1, 1))
    req = np.array([0, 1])
    pos = np.array([0, 0])
    res = _layer(w, b, req=req, pos=pos)
    assert (res["topk"][0, :, 0] == 0).all() and (res["topk"][0, :, 1:] == -1).all()
    assert (res["sparse_ctx"] == 1).all()
    vb = _pages.read_back(w.v_pool.numpy(), 1, "v")
    for t in range(2):
        page = int(w.block_table[req[t], 0]) * 8
        v0 = torch.from_numpy(vb[page].reshape(-1).copy()).view(torch.float8_e4m3fn).double().reshape(16, 128)[0]
        np.testing.assert_allclose(res["out"][t], np.broadcast_to(v0.numpy() * w.v_scale, (16, 128)),
                                   rtol=1e-12, atol=0)
