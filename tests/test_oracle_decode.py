"""Pins for the oracle's four decode steps (CPU only).

Each step is checked against something other than its own code: pure-Python
brute force on tiny inputs, closed forms (one-token blocks, one-token rows,
equal keys), a library routine on the special case it reduces to (dense causal
attention by torch's scaled_dot_product_attention when every block is
selected), and invariants the sources state (the tail block is always selected,
pad rows compute nothing, one page id addresses K and V).
"""
import math

import numpy as np
import pytest
import torch

from indexer_selected_block_amd import workload as wl
from oracle import decode as od
from oracle import formats, pools

import _pages


# ------------------------------------------------------------------ helpers
def _index_pages(t):
    """[n, 128 tok, 128 dim] bf16/e4m3 tensor -> index pages: 8 tiles of 16 keys,
    each laid out lane by lane like a K page."""
    n = t.shape[0]
    e = t.element_size()
    raw = t.contiguous().view(torch.uint8).numpy().reshape(n * 8, 16, 128, e)
    return _pages.k_pages(raw).reshape(n, -1)


def _fp8_index_pool(rng, nblocks):
    vals = torch.from_numpy(rng.standard_normal((nblocks, 128, 128)).astype(np.float32) * 8)
    e4 = vals.to(torch.float8_e4m3fn)
    return _index_pages(e4), e4.double().numpy()


def _bf16_index_pool(rng, nblocks):
    vals = torch.from_numpy(rng.standard_normal((nblocks, 128, 128)).astype(np.float32))
    b = vals.to(torch.bfloat16)
    return _index_pages(b), b.double().numpy()


def _brute_scores(keys_by_block, q_idx, block_table, seq_lens, q_len, H_kv, MB, idx_scale=1.0):
    """Pure-Python loops over tokens, dims and heads."""
    T, H_idx, D = q_idx.shape
    per = H_idx // H_kv
    out = [[[-math.inf] * MB for _ in range(T)] for _ in range(H_kv)]
    for t in range(T):
        r, i = divmod(t, q_len)
        Lt = max(0, int(seq_lens[r]) - (q_len - 1 - i))
        for b in range(MB):
            if 128 * b >= Lt:
                continue
            for g in range(H_kv):
                total = 0.0
                for h in range(g * per, (g + 1) * per):
                    best = -math.inf
                    for j in range(128):
                        if 128 * b + j >= Lt:
                            break
                        k = keys_by_block[int(block_table[r][b])][j]
                        dot = 0.0
                        for d in range(D):
                            dot += float(q_idx[t, h, d]) * float(k[d]) * idx_scale
                        best = max(best, dot)
                    total += best
                out[g][t][b] = total
    return np.array(out)


# ------------------------------------------------------------------ index score
@pytest.mark.parametrize("H_idx,H_kv,q_len", [(1, 1, 1), (2, 1, 2), (2, 2, 3)])
def test_index_score_brute_force_tiny(H_idx, H_kv, q_len):
    rng = np.random.default_rng(11 + H_idx + q_len)
    pool, keys = _fp8_index_pool(rng, 6)
    seq_lens = np.array([130, 0, 257])[: 3]
    bt = np.array([[4, 1, 5], [5, 5, 5], [0, 3, 2]])
    T = 3 * q_len
    q_idx = rng.standard_normal((T, H_idx, 128))
    got = od.index_score(q_idx, pool, "fp8", 0.25, bt, seq_lens, q_len, H_kv, 3)
    ref = _brute_scores(keys, q_idx, bt, seq_lens, q_len, H_kv, 3, idx_scale=0.25)
    assert got.shape == (H_kv, T, 3)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_index_score_brute_force_prefill_chunk():
    # A 20-token chunk at the end of a 140-token request: token i's causal
    # length is 121 + i, so tokens 0..7 see block 0 only (block 1 is -inf for
    # them) and tokens 8..19 see 1..12 keys of block 1; two index heads summed.
    rng = np.random.default_rng(21)
    pool, keys = _fp8_index_pool(rng, 3)
    seq_lens = np.array([140])
    bt = np.array([[2, 0]])
    q_len, H_idx, H_kv = 20, 2, 1
    q_idx = rng.standard_normal((q_len, H_idx, 128))
    got = od.index_score(q_idx, pool, "fp8", 0.5, bt, seq_lens, q_len, H_kv, 2)
    ref = _brute_scores(keys, q_idx, bt, seq_lens, q_len, H_kv, 2, idx_scale=0.5)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.isneginf(got[0, :8, 1]).all() and np.isfinite(got[0, 8:, 1]).all()
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_index_score_one_token_equals_dot():
    rng = np.random.default_rng(3)
    pool, keys = _bf16_index_pool(rng, 2)
    q_idx = rng.standard_normal((1, 1, 128))
    got = od.index_score(q_idx, pool, "bf16", 1.0, np.array([[1, 0]]), np.array([1]), 1, 1, 2)
    assert got[0, 0, 0] == pytest.approx(float(np.dot(keys[1, 0], q_idx[0, 0])), rel=1e-13)
    assert got[0, 0, 1] == -np.inf


def test_index_score_full_blocks_is_blockwise_max():
    rng = np.random.default_rng(4)
    pool, keys = _bf16_index_pool(rng, 4)
    q_idx = rng.standard_normal((1, 1, 128))
    bt = np.array([[2, 0, 3]])
    got = od.index_score(q_idx, pool, "bf16", 1.0, bt, np.array([384]), 1, 1, 3)
    ref = np.einsum("btd,d->bt", keys[[2, 0, 3]], q_idx[0, 0]).max(axis=1)
    np.testing.assert_allclose(got[0, 0], ref, rtol=1e-13)


def test_index_score_is_causal_per_query_token():
    rng = np.random.default_rng(5)
    vals = torch.from_numpy(rng.standard_normal((2, 128, 128)).astype(np.float32)).to(torch.bfloat16)
    L = 129                                     # token 0 of 2 sees 128 keys, token 1 sees 129
    # poison the key at position 128 (block 1, slot 0): only token 1 may read it
    vals[1, 0, :] = float("nan")
    bad = _index_pages(vals)
    q_idx = rng.standard_normal((2, 1, 128))
    s = od.index_score(q_idx, bad, "bf16", 1.0, np.array([[0, 1]]), np.array([L]), 2, 1, 2)
    assert np.isfinite(s[0, 0, 0]) and s[0, 0, 1] == -np.inf     # token 0: one block
    assert np.isfinite(s[0, 1, 0]) and np.isnan(s[0, 1, 1])      # token 1 reads the poison


def test_index_score_sums_the_heads_of_a_group():
    rng = np.random.default_rng(6)
    pool, _ = _fp8_index_pool(rng, 3)
    q1 = rng.standard_normal((2, 1, 128))
    q2 = np.concatenate([q1, q1], axis=1)                        # two identical heads
    bt = np.array([[2, 1], [0, 2]])
    lens = np.array([200, 77])
    s1 = od.index_score(q1, pool, "fp8", 1.0, bt, lens, 1, 1, 2)
    s2 = od.index_score(q2, pool, "fp8", 1.0, bt, lens, 1, 1, 2)
    fin = np.isfinite(s1)
    np.testing.assert_allclose(s2[fin], 2 * s1[fin], rtol=1e-13)
    s3 = od.index_score(q2, pool, "fp8", 1.0, bt, lens, 1, 2, 2)   # one head per KV group
    np.testing.assert_allclose(s3[0][fin[0]], s1[0][fin[0]], rtol=1e-13)
    np.testing.assert_allclose(s3[1][fin[0]], s1[0][fin[0]], rtol=1e-13)


def test_index_score_relabelling_pages_changes_nothing():
    rng = np.random.default_rng(7)
    pool, _ = _fp8_index_pool(rng, 5)
    perm = rng.permutation(5)
    inv = np.argsort(perm)
    pool2 = pool[perm]                     # block b now sits at physical id inv[b]
    bt = np.array([[3, 0, 4], [1, 2, 0]])
    q_idx = rng.standard_normal((2, 1, 128))
    lens = np.array([300, 256])
    a = od.index_score(q_idx, pool, "fp8", 1.0, bt, lens, 1, 1, 3)
    b = od.index_score(q_idx, pool2, "fp8", 1.0, inv[bt], lens, 1, 1, 3)
    assert np.array_equal(a, b)


def test_index_score_mxfp4_against_brute_force():
    cfg = wl.shrink(wl.CONFIGS["mxfp4"], num_reqs=2, ctx_lo=150, ctx_hi=260)
    w = wl.make_workload(cfg)
    pool = w.idx_pool.numpy()
    keys = {b: formats.decode_mxfp4_page(pool[b]) for b in range(pool.shape[0])}
    q_idx = formats.decode_e4m3(w.q_idx.numpy())
    bt, lens = w.block_table.numpy(), w.seq_lens.numpy()
    got = od.index_score(q_idx, pool, "mxfp4", 1.0, bt, lens, 1, 1, cfg.max_blocks)
    ref = _brute_scores(keys, q_idx, bt, lens, 1, 1, cfg.max_blocks)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12)


# ------------------------------------------------------------------ top-k
def _brute_topk_row(s, nt, K):
    """Sort with Python's sorted(): non-NaN first, score descending, index ascending."""
    if nt == 0:
        return [-1] * K
    tail = nt - 1
    ranked = sorted(range(tail), key=lambda b: (math.isnan(s[b]), -(0.0 if math.isnan(s[b]) else s[b]), b))
    sel = sorted(ranked[: min(K - 1, tail)] + [tail])
    return sel + [-1] * (K - len(sel))


@pytest.mark.parametrize("K", [1, 2, 3, 5, 8, 40])
def test_topk_brute_force_with_ties_and_specials(K):
    rng = np.random.default_rng(K)
    q_len, R, MB = 2, 9, 20
    lens = rng.integers(0, MB * 128 + 1, R)
    lens[0], lens[1] = 0, 1
    palette = np.array([0.5, -0.0, 0.0, 1.0, np.inf, -np.inf, np.nan, 3.0, -2.0], dtype=np.float32)
    scores = palette[rng.integers(0, len(palette), (2, R * q_len, MB))]
    got = od.topk_select(scores, lens, q_len, K)
    for g in range(2):
        for t in range(R * q_len):
            r, i = divmod(t, q_len)
            nt = od.num_blocks(od.causal_length(lens[r], q_len, i))
            assert list(got[g, t]) == _brute_topk_row(list(map(float, scores[g, t])), nt, K)


def test_topk_special_values_order():
    s = np.array([[[np.nan, -np.inf, -0.0, 0.0, -1e30, 7.0]]], dtype=np.float32)
    # 6 blocks -> tail 5 forced; the best two of blocks 0..4 are -0.0 (block 2) and
    # +0.0 (block 3): equal, so both beat -1e30; NaN ranks below -inf.
    assert list(od.topk_select(s, [6 * 128], 1, 3)[0, 0]) == [2, 3, 5]
    assert list(od.topk_select(s, [6 * 128], 1, 5)[0, 0]) == [1, 2, 3, 4, 5]
    assert list(od.topk_select(s, [6 * 128], 1, 6)[0, 0]) == [0, 1, 2, 3, 4, 5]
    assert list(od.topk_select(s, [6 * 128], 1, 1)[0, 0]) == [5]


def test_topk_invariants_on_random_rows():
    rng = np.random.default_rng(9)
    R, q_len, MB, K = 30, 3, 64, 16
    lens = rng.integers(0, MB * 128 + 1, R)
    scores = rng.standard_normal((1, R * q_len, MB)).astype(np.float32)
    out = od.topk_select(scores, lens, q_len, K)
    for t in range(R * q_len):
        r, i = divmod(t, q_len)
        nt = od.num_blocks(od.causal_length(lens[r], q_len, i))
        sel = [b for b in out[0, t] if b >= 0]
        assert len(sel) == min(K, nt)                        # |S| = min(K, n_t)
        assert all(out[0, t, len(sel):] == -1)
        assert sel == sorted(set(sel))                       # ascending, distinct
        if nt:
            assert sel[-1] == nt - 1                         # the tail is always selected
            if K >= nt:
                assert sel == list(range(nt))                # K >= n_t keeps every block
            else:
                worst = min(scores[0, t, b] for b in sel[:-1]) if K > 1 else np.inf
                rest = [scores[0, t, b] for b in range(nt - 1) if b not in sel]
                assert all(x <= worst for x in rest)


# ------------------------------------------------------------------ emit
@pytest.mark.parametrize("ppb", [8, 1])
def test_emit_pages_and_lengths(ppb):
    rng = np.random.default_rng(10 + ppb)
    R, q_len, MB, K, H_kv = 7, 4, 12, 5, 2
    lens = rng.integers(0, MB * 128 + 1, R)
    lens[2] = 0
    lens[3] = 2                                              # shorter than q: some rows empty
    bt = rng.integers(0, 50, (R, MB))
    scores = rng.standard_normal((H_kv, R * q_len, MB))
    topk = od.topk_select(scores, lens, q_len, K)
    sbt, sctx = od.emit_sparse_block_table(topk, bt, lens, q_len, H_kv, K, ppb)
    assert sbt.shape == (R * q_len * H_kv, K * ppb)
    for t in range(R * q_len):
        r, i = divmod(t, q_len)
        Lt = od.causal_length(lens[r], q_len, i)
        for g in range(H_kv):
            row = t * H_kv + g
            sel = [b for b in topk[g, t] if b >= 0]
            # sparse length by counting the causal positions whose block is selected
            assert sctx[row] == sum(1 for p in range(Lt) if p // 128 in sel)
            want = [bt[r][b] * ppb + p for b in sel for p in range(ppb)]
            assert list(sbt[row, : len(want)]) == want
            assert all(sbt[row, len(want):] == -1)


def test_emit_page_ids_address_k_and_v():
    # One page id addresses a K page and a V page (vLLM PR 61889, Details); the
    # pools are separate and equally long, so the printed K/V row mismatch
    # (890768 vs 890760) cannot arise and every emitted id is in both.
    for name in ("tiny_bf16", "long_context"):
        cfg = wl.shrink(wl.CONFIGS[name], num_reqs=3, ctx_lo=200, ctx_hi=700)
        w = wl.make_workload(cfg)
        assert w.k_pool.shape == w.v_pool.shape
        lens, bt = w.seq_lens.numpy(), w.block_table.numpy()
        scores = np.random.default_rng(1).standard_normal((1, cfg.num_tokens, cfg.max_blocks))
        topk = od.topk_select(scores, lens, cfg.query_len, cfg.top_k)
        sbt, _ = od.emit_sparse_block_table(topk, bt, lens, cfg.query_len, 1, cfg.top_k,
                                            cfg.pages_per_block)
        ids = sbt[sbt >= 0]
        assert ids.max() < w.k_pool.shape[0] and ids.max() < w.v_pool.shape[0]
        assert ids.max() <= (cfg.pool_blocks + 1) * cfg.pages_per_block - 1


# ------------------------------------------------------------------ attention
def _kv_pools_fp8(rng, npages, kscale, vscale):
    k = torch.from_numpy(rng.standard_normal((npages, 16, 128)).astype(np.float32)).to(torch.float8_e4m3fn)
    v = torch.from_numpy(rng.standard_normal((npages, 16, 128)).astype(np.float32)).to(torch.float8_e4m3fn)
    kp = _pages.k_pages(k.view(torch.uint8).numpy().reshape(npages, 16, 128, 1))
    vp = _pages.v_pages(v.view(torch.uint8).numpy().reshape(npages, 16, 128, 1))
    return kp, vp, k.double().numpy() * kscale, v.double().numpy() * vscale


def test_attention_one_token_row_returns_v0():
    rng = np.random.default_rng(12)
    kp, vp, K, V = _kv_pools_fp8(rng, 4, 0.5, 2.0)
    q = rng.standard_normal((1, 4, 128))
    sbt = np.array([[3, 1]])
    out = od.sparse_pa_decode(q, kp, vp, "fp8", 0.5, 2.0, sbt, np.array([1]), 1, 8, 0.1)
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], V[3, 0])


def test_attention_equal_keys_give_mean_v_and_empty_rows_zero():
    rng = np.random.default_rng(13)
    kp, vp, K, V = _kv_pools_fp8(rng, 3, 1.0, 1.0)
    same = np.repeat(K[0, :1] / 1.0, 16, axis=0)                         # every key = key 0 of page 0
    kp[:] = _pages.k_pages(torch.from_numpy(np.stack([same] * 3)).to(torch.float8_e4m3fn)
                           .view(torch.uint8).numpy().reshape(3, 16, 128, 1))
    q = rng.standard_normal((2, 2, 128))
    sbt = np.array([[2, 0, -1], [1, 1, 1]])
    sctx = np.array([20, 0])
    out = od.sparse_pa_decode(q, kp, vp, "fp8", 1.0, 1.0, sbt, sctx, 1, 8, 0.3)
    want = np.concatenate([V[2], V[0]])[:20].mean(axis=0)
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-12, atol=1e-14)
    assert np.all(out[1] == 0)


def _dense_reference(w):
    """Dense causal attention over every position < L_t with torch SDPA (float64),
    K/V decoded by torch's own views of the page bytes."""
    cfg = w.cfg
    q = w.q.view(torch.bfloat16).double() if cfg.q_dtype == "bf16" else w.q.view(torch.float8_e4m3fn).double()
    T, Hq = q.shape[0], cfg.num_q_heads
    out = torch.zeros(T, Hq, 128, dtype=torch.float64)
    ppb = cfg.pages_per_block
    assert cfg.kv_dtype in ("fp8", "bf16")
    view = torch.float8_e4m3fn if cfg.kv_dtype == "fp8" else torch.bfloat16
    e = 1 if cfg.kv_dtype == "fp8" else 2
    kb = _pages.read_back(w.k_pool.numpy(), e, "k")
    vb = _pages.read_back(w.v_pool.numpy(), e, "v")
    kpages = torch.from_numpy(kb.reshape(kb.shape[0], -1).copy()).view(view).double().reshape(-1, 16, 128)
    vpages = torch.from_numpy(vb.reshape(vb.shape[0], -1).copy()).view(view).double().reshape(-1, 16, 128)
    kpages = kpages * (w.k_scale if cfg.kv_dtype == "fp8" else 1)
    vpages = vpages * (w.v_scale if cfg.kv_dtype == "fp8" else 1)
    for t in range(T):
        r, i = divmod(t, cfg.query_len)
        Lt = od.causal_length(int(w.seq_lens[r]), cfg.query_len, i)
        if Lt == 0:
            continue
        pos = torch.arange(Lt)
        page = w.block_table[r, pos // 128].long() * ppb + (pos % 128) // 16
        K = kpages[page, pos % 16]
        V = vpages[page, pos % 16]
        o = torch.nn.functional.scaled_dot_product_attention(
            q[t].reshape(1, Hq, 1, 128), K.expand(1, Hq, Lt, 128), V.expand(1, Hq, Lt, 128),
            scale=w.sm_scale)
        out[t] = o.reshape(Hq, 128)
    return out.numpy()


@pytest.mark.parametrize("name", ["tiny_bf16", "spec_decode"])
def test_layer_with_every_block_selected_is_dense_attention(name):
    base = wl.CONFIGS[name]
    cfg = wl.shrink(base, num_reqs=3, ctx_lo=100, ctx_hi=900, num_pad_reqs=1,
                    top_k=8)                                    # 8 blocks >= n_t everywhere
    w = wl.make_workload(cfg)
    q = formats.decode_query(w.q.numpy(), cfg.q_dtype)
    q_idx = formats.decode_query(w.q_idx.numpy(), cfg.qidx_dtype)
    res = od.decode_layer(q, q_idx, w.idx_pool.numpy(), cfg.idx_dtype, w.idx_scale,
                          w.k_pool.numpy(), w.v_pool.numpy(), cfg.kv_dtype, w.k_scale, w.v_scale,
                          w.block_table.numpy(), w.seq_lens.numpy(), cfg.query_len,
                          cfg.num_kv_heads, cfg.max_blocks, cfg.top_k, cfg.pages_per_block,
                          w.sm_scale)
    dense = _dense_reference(w)
    assert np.isfinite(res["out"]).all()
    np.testing.assert_allclose(res["out"], dense, rtol=1e-10, atol=1e-12)
    # pad rows (length 0) select nothing and output zeros
    lens = w.seq_lens.numpy()
    for t in range(cfg.num_tokens):
        r, i = divmod(t, cfg.query_len)
        if od.causal_length(lens[r], cfg.query_len, i) == 0:
            assert (res["topk"][:, t] == -1).all() and res["sparse_ctx"][t] == 0
            assert (res["out"][t] == 0).all()


def test_attention_mxfp4_pages_match_dense_on_decoded_values():
    cfg = wl.shrink(wl.CONFIGS["mxfp4"], num_reqs=2, ctx_lo=130, ctx_hi=400, top_k=4)
    w = wl.make_workload(cfg)
    kp, vp = w.k_pool.numpy(), w.v_pool.numpy()
    q = formats.decode_e4m3(w.q.numpy())
    lens, bt = w.seq_lens.numpy(), w.block_table.numpy()
    topk = od.topk_select(np.zeros((1, 2, cfg.max_blocks)), lens, 1, 4)
    sbt, sctx = od.emit_sparse_block_table(topk, bt, lens, 1, 1, 4, 1)
    out = od.sparse_pa_decode(q, kp, vp, "mxfp4", 1.0, 1.0, sbt, sctx, 1, 1, w.sm_scale)
    for t in range(2):
        L = int(lens[t])
        K = np.concatenate([formats.decode_mxfp4_page(kp[b]) for b in bt[t][: -(-L // 128)]])[:L]
        V = np.concatenate([formats.decode_mxfp4_page(vp[b]) for b in bt[t][: -(-L // 128)]])[:L]
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[t]).reshape(1, 16, 1, 128),
            torch.from_numpy(K).expand(1, 16, L, 128), torch.from_numpy(V).expand(1, 16, L, 128),
            scale=w.sm_scale)
        np.testing.assert_allclose(out[t], o.reshape(16, 128).numpy(), rtol=1e-10, atol=1e-12)


def test_shard_selections_merged_give_the_whole_row_selection():
    # The context-parallel reading: each shard of a row's blocks selects as if
    # it were a whole row; the top K - 1 of the union of the shards' picks
    # (excluding the row's tail), plus the tail, is the whole row's selection.
    import math

    def order(sc, b):                       # larger first, NaN last, -0 == +0, then lower index
        s = float(sc)
        return (1, 0.0, b) if math.isnan(s) else (0, -(s + 0.0), b)

    rng = np.random.default_rng(12)
    for trial in range(300):
        n = int(rng.integers(2, 90))
        K = int(rng.integers(1, 12))
        row = rng.choice([-1.0, -0.0, 0.0, 0.5, 1.0, np.nan, np.inf, -np.inf], size=n) if trial % 3 == 0 \
            else np.round(rng.standard_normal(n), 1)
        row = row.astype(np.float32)
        whole = od.topk_select(row[None, None, :], np.array([n * 128]), 1, K)[0, 0]
        G = int(rng.integers(1, min(n, 6) + 1))
        cuts = np.sort(rng.choice(np.arange(1, n), size=G - 1, replace=False)) if G > 1 else np.array([], int)
        bounds = np.concatenate([[0], cuts, [n]])
        cands = set()
        for a, b in zip(bounds[:-1], bounds[1:]):
            sel = od.topk_select(row[None, None, a:b], np.array([(b - a) * 128]), 1, K)[0, 0]
            cands |= {a + int(x) for x in sel if x >= 0}
        tail = n - 1
        pool = sorted((c for c in cands if c != tail), key=lambda c: order(row[c], c))
        merged = sorted(pool[:K - 1] + [tail])
        want = [int(x) for x in whole if x >= 0]
        assert merged == want, (trial, n, K, G, merged, want)


def test_merge_candidates_of_shards_equals_the_whole_row_selection():
    rng = np.random.default_rng(13)
    for trial in range(40):
        H, T, MB = 2, 6, int(rng.integers(2, 200))
        K = int(rng.integers(1, 20))
        if trial % 2:
            scores = rng.choice([-1.0, -0.0, 0.0, 0.5, np.nan, np.inf, -np.inf], size=(H, T, MB)).astype(np.float32)
        else:
            scores = np.round(rng.standard_normal((H, T, MB)), 1).astype(np.float32)
        lens = rng.integers(0, MB * 128 + 1, T)
        lens[0] = 0
        G = int(rng.integers(1, 7))
        from _util import shard_candidates
        sc, ids = shard_candidates(scores, lens, G, K, rng)
        merged = od.merge_candidates(sc, ids, lens, 1, K, MB)
        assert np.array_equal(merged, od.topk_select(scores, lens, 1, K)), trial
