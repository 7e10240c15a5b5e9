"""GPU parity: every call of libisb against the CPU oracle (needs an MI355X).

* Per call, on shrunk workloads of all five configurations (several tiles,
  ragged tails, pad rows): scores within 1e-3 relative; top-k and block
  tables bit-exact when both sides get the same fp32 scores / the same
  selection; attention within 1e-2 max|V| + 1e-3 (fp8, MXFP4) or
  4e-3 max|V| (bf16).
* The chained layer, every row: the oracle's top-k of the GPU's own fp32
  scores equals the GPU's selection bit for bit, the oracle's emit of it
  equals the GPU's table, and the oracle's attention over the GPU's table
  matches the GPU's output; the GPU's selection is also a valid top-k of the
  oracle's fp64 scores within the GPU's score error.
* Full-size workloads in the launch configuration the benchmark times, on
  sampled requests the oracle recomputes from their own pages.
"""
import dataclasses

import numpy as np
import pytest
import torch

import indexer_selected_block_amd as isb
from indexer_selected_block_amd import workload as wl
from oracle import decode as od

from _util import (assert_scores_close, attn_tol, attended_vmax, check_chain, host_inputs, oracle_attention,
                   oracle_layer, oracle_scores, sample_requests, small_configs)

pytestmark = pytest.mark.gpu

SMALL = small_configs()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    isb.load_library()


_cache = {}


def _run_small(name):
    if name not in _cache:
        w = wl.make_workload(SMALL[name], device="cuda")
        layer = isb.DecodeLayer(w)
        layer.run()
        torch.cuda.synchronize()
        _cache[name] = (w, layer, host_inputs(w))
    return _cache[name]


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ index score
@pytest.mark.parametrize("name", list(SMALL))
def test_index_score_parity(name):
    _say(f"[index_score] {name}")
    w, layer, hi = _run_small(name)
    assert_scores_close(layer.scores.cpu().numpy(), oracle_scores(hi))


def test_index_score_output_contents_do_not_matter():
    w, layer, hi = _run_small("spec_decode")
    cfg = w.cfg
    a = torch.full_like(layer.scores, float("nan"))
    b = torch.zeros_like(layer.scores)
    for buf in (a, b):
        isb.index_score(w.q_idx, cfg.qidx_dtype, w.idx_pool, cfg.idx_dtype, w.idx_scale, w.block_table,
                        w.seq_lens, cfg.query_len, cfg.num_kv_heads, cfg.max_blocks, scores=buf)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), layer.scores.view(torch.int32))


def test_index_score_two_kv_heads_and_bf16_query_on_mxfp4():
    # H_kv = 2 with 4 index heads (2 per group); MXFP4 keys with a bf16 index query
    # take the bf16 tile path; e4m3 query on fp8 keys takes the converted tile path.
    for base, kw in ((wl.CONFIGS["mxfp4"], dict(qidx_dtype="bf16")),
                     (wl.CONFIGS["spec_decode"], dict(qidx_dtype="e4m3", num_idx_heads=2)),
                     (wl.CONFIGS["mxfp4"], dict(num_kv_heads=2, num_q_heads=16))):
        cfg = dataclasses.replace(wl.shrink(base, num_reqs=3, ctx_lo=200, ctx_hi=1400), **kw)
        _say(f"[index_score variant] {cfg.name} {kw}")
        w = wl.make_workload(cfg, device="cuda")
        s = isb.index_score(w.q_idx, cfg.qidx_dtype, w.idx_pool, cfg.idx_dtype, w.idx_scale,
                            w.block_table, w.seq_lens, cfg.query_len, cfg.num_kv_heads, cfg.max_blocks)
        torch.cuda.synchronize()
        assert_scores_close(s.cpu().numpy(), oracle_scores(host_inputs(w)))


WIDE_CASES = {
    # more than 16 tokens or 64 index rows a request: the wide scorer, for every
    # key / index-query type pair and head layout (index heads per KV group 1..4,
    # 16-row tiles holding 1..16 tokens), each with a ragged last query tile
    "fp8_bf16q_8heads_2kv": ("spec_decode", dict(query_len=24, num_idx_heads=8, num_kv_heads=2)),
    "fp8_e4m3q": ("spec_decode", dict(query_len=33, qidx_dtype="e4m3")),
    "mxfp4_e4m3q_16heads_4kv": ("mxfp4", dict(query_len=9, num_idx_heads=16, num_kv_heads=4)),
    "mxfp4_bf16q": ("mxfp4", dict(query_len=20, qidx_dtype="bf16")),
    "bf16_e4m3q_2heads_2kv": ("tiny_bf16", dict(query_len=40, num_idx_heads=2, num_kv_heads=2,
                                                qidx_dtype="e4m3")),
}


@pytest.mark.parametrize("case", list(WIDE_CASES))
def test_index_score_wide_variants(case):
    base, kw = WIDE_CASES[case]
    cfg = dataclasses.replace(wl.shrink(wl.CONFIGS[base], num_reqs=3, ctx_lo=300, ctx_hi=1400, num_pad_reqs=0),
                              **kw)
    assert cfg.query_len > 16 or cfg.query_len * cfg.num_idx_heads > 64
    _say(f"[index_score wide] {case}")
    w = wl.make_workload(cfg, device="cuda")
    s = isb.index_score(w.q_idx, cfg.qidx_dtype, w.idx_pool, cfg.idx_dtype, w.idx_scale,
                        w.block_table, w.seq_lens, cfg.query_len, cfg.num_kv_heads, cfg.max_blocks)
    torch.cuda.synchronize()
    assert_scores_close(s.cpu().numpy(), oracle_scores(host_inputs(w)))


# ------------------------------------------------------------------ top-k
def _adversarial_scores(rng, H_kv, T, MB, K):
    palette = np.array([0.5, -0.0, 0.0, 1.0, np.inf, -np.inf, np.nan, 3.0, -2.0, 1e-30, -1e30],
                       dtype=np.float32)
    s = rng.standard_normal((H_kv, T, MB)).astype(np.float32)
    tie_rows = rng.random((H_kv, T)) < 0.5
    pal = palette[rng.integers(0, len(palette), (H_kv, T, MB))]
    s[tie_rows] = pal[tie_rows]
    return s


def _lengths_covering(rng, R, q_len, MB, K):
    # causal block counts 0, 1, K-1, K, K+1 and MB all occur
    special = [0, 1, 128 * (K - 1), 128 * K, 128 * K + 1, 128 * MB, 128 * (K + 1) + 5, 127]
    lens = rng.integers(0, 128 * MB + 1, R)
    lens[: min(R, len(special))] = [min(x, 128 * MB) for x in special[:R]]
    return lens.astype(np.int32)


@pytest.mark.parametrize("q_len,H_kv", [(1, 1), (4, 1), (2, 2)])
@pytest.mark.parametrize("K", [1, 2, 7, 16, 32])
def test_topk_bit_exact(K, q_len, H_kv):
    rng = np.random.default_rng(1000 + K * 10 + q_len + H_kv)
    MB, R = max(K + 3, 48), 24
    lens = _lengths_covering(rng, R, q_len, MB, K)
    s = _adversarial_scores(rng, H_kv, R * q_len, MB, K)
    ref = od.topk_select(s, lens, q_len, K)
    got = isb.topk_select(torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), q_len, K)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("MB,R,q_len,K", [(8192, 8, 2, 32), (256, 1075, 4, 16), (512, 128, 1, 16),
                                          (1024, 64, 1, 16), (10000, 4, 1, 32), (3000, 6, 1, 5),
                                          (1027, 5, 1, 16), (4095, 3, 2, 32)])
def test_topk_full_size_shapes(MB, R, q_len, K):
    _say(f"[topk] MB={MB} rows={R * q_len}")
    rng = np.random.default_rng(MB + R)
    lens = rng.integers(0, 128 * MB + 1, R).astype(np.int32)
    lens[0] = 128 * MB
    lens[1] = 0
    s = rng.standard_normal((1, R * q_len, MB)).astype(np.float32)
    s[0, :, ::7] = np.round(s[0, :, ::7])          # plenty of exact ties
    ref = od.topk_select(s, lens, q_len, K)
    got = isb.topk_select(torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), q_len, K)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def _shared_prefix_rows(rng, rows, MB):
    """Score rows whose candidates share long runs of leading key bits (the
    selection starts below them on wide rows): all equal; equal but for the
    lowest three mantissa bits; two exponents; equal with NaNs and a few one
    ulp above; mostly -inf; standard normal (signs differ: no shared bits)."""
    s = np.empty((rows, MB), np.float32)
    for r in range(rows):
        kind = r % 6
        if kind == 0:
            s[r] = 2.5
        elif kind == 1:
            s[r] = (np.uint32(0x3F800000) + rng.integers(0, 8, MB).astype(np.uint32)).view(np.float32)
        elif kind == 2:
            s[r] = rng.choice(np.array([3.0, 3.5, 5.0, 6.0], np.float32), MB)
        elif kind == 3:
            s[r] = 7.0
            s[r, rng.integers(0, MB, 5)] = np.nan
            s[r, rng.integers(0, MB, 3)] = np.nextafter(np.float32(7.0), np.float32(8.0))
        elif kind == 4:
            s[r] = -np.inf
            s[r, rng.integers(0, MB, 40)] = -1.0
        else:
            s[r] = rng.standard_normal(MB)
    return s


@pytest.mark.parametrize("MB,K", [(1024, 16), (2048, 16), (4096, 32), (8192, 32)])
def test_topk_rows_sharing_leading_bits(MB, K):
    rng = np.random.default_rng(MB + K)
    R = 12
    lens = np.full(R, 128 * MB, np.int32)
    lens[6:] = rng.integers(128 * (MB // 2), 128 * MB + 1, R - 6)
    s = _shared_prefix_rows(rng, R, MB)[None]
    ref = od.topk_select(s, lens, 1, K)
    got = isb.topk_select(torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), 1, K)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("case", ["mxfp4_3904_blocks", "long_context_4096_blocks", "long_context_8192_blocks"])
def test_select_attend_rows_sharing_leading_bits(case):
    # The selection inside the attention launch on the same rows, against the
    # oracle's selection (and the two-call path's page table and output).
    base, kw = _SEL_CASES[case]
    cfg = dataclasses.replace(SMALL[base], **kw)
    w = wl.make_workload(cfg, device="cuda")
    T, H_kv, MB = cfg.num_tokens, cfg.num_kv_heads, cfg.max_blocks
    rng = np.random.default_rng(MB)
    s = _shared_prefix_rows(rng, H_kv * T, MB).reshape(H_kv, T, MB)
    scores = torch.from_numpy(s).cuda()
    ref = od.topk_select(s, w.seq_lens.cpu().numpy(), cfg.query_len, cfg.top_k)
    topk, sbt, sctx = isb.topk_select_emit(scores, w.seq_lens, cfg.query_len, cfg.top_k, w.block_table,
                                           cfg.pages_per_block)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               sbt, sctx, cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale,
                               decode_query_len=cfg.query_len)
    f_topk = torch.full_like(topk, 777)
    f_sbt = torch.full_like(sbt, -5)
    f_sctx = torch.full_like(sctx, 3)
    f_out = torch.full_like(out, float("nan"))
    isb.select_attend(scores, w.seq_lens, cfg.query_len, cfg.top_k, w.block_table, w.q, cfg.q_dtype, w.k_pool,
                      w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, cfg.num_q_heads, w.sm_scale,
                      topk_idx=f_topk, sparse_bt=f_sbt, sparse_ctx=f_sctx, out=f_out)
    torch.cuda.synchronize()
    assert np.array_equal(topk.cpu().numpy(), ref)
    assert np.array_equal(f_topk.cpu().numpy(), ref)
    assert torch.equal(f_sbt, sbt) and torch.equal(f_sctx, sctx)
    assert torch.equal(f_out.view(torch.int16), out.view(torch.int16))


# ------------------------------------------------------------------ emit
@pytest.mark.parametrize("ppb", [8, 1])
@pytest.mark.parametrize("H_kv,q_len", [(1, 1), (1, 4), (2, 3)])
def test_emit_bit_exact(ppb, H_kv, q_len):
    rng = np.random.default_rng(ppb * 7 + H_kv + q_len)
    R, MB, K = 19, 40, 9
    lens = _lengths_covering(rng, R, q_len, MB, K)
    bt = rng.integers(0, 5000, (R, MB)).astype(np.int32)
    topk = od.topk_select(rng.standard_normal((H_kv, R * q_len, MB)), lens, q_len, K)
    sbt, sctx = od.emit_sparse_block_table(topk, bt, lens, q_len, H_kv, K, ppb)
    g_sbt, g_sctx = isb.emit_sparse_block_table(torch.from_numpy(topk).cuda(), torch.from_numpy(bt).cuda(),
                                                torch.from_numpy(lens).cuda(), q_len, ppb)
    torch.cuda.synchronize()
    assert np.array_equal(g_sbt.cpu().numpy(), sbt)
    assert np.array_equal(g_sctx.cpu().numpy(), sctx)


# ------------------------------------------------------------------ fused top-k + emit
# Widths cover each launch shape of the fused call: 256-thread rows with the
# block-table row in LDS, 1024-thread rows that read only the selected
# entries of it, and rows too wide for LDS (two launches).
@pytest.mark.parametrize("MB,R,q_len,H_kv,K,ppb", [(48, 24, 1, 1, 7, 8), (40, 19, 3, 2, 9, 1),
                                                   (512, 40, 1, 1, 16, 8), (3000, 6, 2, 1, 32, 8),
                                                   (8192, 4, 2, 1, 32, 8), (10000, 3, 1, 2, 16, 1),
                                                   (300, 5, 4, 1, 300, 8), (45, 7, 1, 1, 5, 8),
                                                   (1027, 4, 1, 1, 16, 1)])
def test_topk_select_emit_matches_oracle(MB, R, q_len, H_kv, K, ppb):
    _say(f"[topk+emit] MB={MB} R={R} q={q_len} H_kv={H_kv} K={K} ppb={ppb}")
    rng = np.random.default_rng(MB * 3 + K)
    lens = _lengths_covering(rng, R, q_len, MB, K)
    s = _adversarial_scores(rng, H_kv, R * q_len, MB, K).astype(np.float32)
    bt = rng.integers(0, 5000, (R, MB + 3)).astype(np.int32)   # table stride wider than MB
    topk = od.topk_select(s, lens, q_len, K)
    sbt, sctx = od.emit_sparse_block_table(topk, bt, lens, q_len, H_kv, K, ppb)
    # prior contents of the outputs do not matter
    g_topk = torch.full((H_kv, R * q_len, K), 12345, dtype=torch.int32, device="cuda")
    g_sbt = torch.full((R * q_len * H_kv, K * ppb), -7, dtype=torch.int32, device="cuda")
    g_sctx = torch.full((R * q_len * H_kv,), 99, dtype=torch.int32, device="cuda")
    isb.topk_select_emit(torch.from_numpy(s).cuda(), torch.from_numpy(lens).cuda(), q_len, K,
                         torch.from_numpy(bt).cuda(), ppb, topk_idx=g_topk, sparse_bt=g_sbt,
                         sparse_ctx=g_sctx)
    torch.cuda.synchronize()
    assert np.array_equal(g_topk.cpu().numpy(), topk)
    assert np.array_equal(g_sbt.cpu().numpy(), sbt)
    assert np.array_equal(g_sctx.cpu().numpy(), sctx)


# ------------------------------------------------------------------ select + attend
_SEL_CASES = {
    "fp8_decode": ("fp8_decode", {}),
    "spec_decode": ("spec_decode", {}),
    "tiny_bf16": ("tiny_bf16", {}),
    "fp8_two_kv_heads": ("fp8_decode", dict(num_kv_heads=2, num_q_heads=16, num_idx_heads=2)),
    "long_context_rows_not_x4": ("long_context", {}),     # two launches: rows not a multiple of 4
    "mxfp4": ("mxfp4", {}),                               # one launch, 128-token pages
    "mxfp4_two_kv_heads": ("mxfp4", dict(num_kv_heads=2, num_q_heads=16)),
    "mxfp4_bf16_query": ("mxfp4", dict(q_dtype="bf16")),
    "prefill_mxfp4": ("prefill_mxfp4", {}),              # 37 tokens a request, 74 rows
    # 128 one-token rows of 16 blocks: two splits of eight-wave workgroups
    "fp8_decode_eight_waves": ("fp8_decode", dict(num_reqs=128, ctx_lo=1500, ctx_hi=4000, pool_blocks=128 * 32 + 64)),
    # rows wider than 2048 blocks: one launch that reads only the selected
    # blocks' table entries (4096 and 8192 blocks; MXFP4 at 3904)
    "long_context_4096_blocks": ("long_context", dict(num_reqs=2, ctx_lo=400000, ctx_hi=524288,
                                                      pool_blocks=2 * 4096 + 64)),
    "long_context_8192_blocks": ("long_context", dict(num_reqs=2, ctx_lo=900000, ctx_hi=1048576,
                                                      pool_blocks=2 * 8192 + 64)),
    "mxfp4_3904_blocks": ("mxfp4", dict(num_reqs=3, ctx_lo=300000, ctx_hi=499712, pool_blocks=3 * 3904 + 64)),
    # rows wider than 8192 blocks: the two calls (selection over global memory)
    "long_context_10000_blocks": ("long_context", dict(num_reqs=1, ctx_lo=1200000, ctx_hi=1280000,
                                                       pool_blocks=10000 + 64)),
}


@pytest.mark.parametrize("case", list(_SEL_CASES))
def test_select_attend_matches_the_two_calls(case):
    # The one-launch selection + attention writes exactly what
    # topk_select_emit followed by sparse_pa_decode writes.
    base, kw = _SEL_CASES[case]
    cfg = dataclasses.replace(SMALL[base], **kw)
    _say(f"[select_attend] {case}: MB={cfg.max_blocks}")
    w = wl.make_workload(cfg, device="cuda")
    scores = isb.index_score(w.q_idx, cfg.qidx_dtype, w.idx_pool, cfg.idx_dtype, w.idx_scale, w.block_table,
                             w.seq_lens, cfg.query_len, cfg.num_kv_heads, cfg.max_blocks)
    topk, sbt, sctx = isb.topk_select_emit(scores, w.seq_lens, cfg.query_len, cfg.top_k, w.block_table,
                                           cfg.pages_per_block)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               sbt, sctx, cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale,
                               decode_query_len=cfg.query_len)
    T, H_kv = cfg.num_tokens, cfg.num_kv_heads
    f_topk = torch.full_like(topk, 777)
    f_sbt = torch.full_like(sbt, -5)
    f_sctx = torch.full_like(sctx, 3)
    f_out = torch.full_like(out, float("nan"))
    isb.select_attend(scores, w.seq_lens, cfg.query_len, cfg.top_k, w.block_table, w.q, cfg.q_dtype, w.k_pool,
                      w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, cfg.num_q_heads, w.sm_scale,
                      topk_idx=f_topk, sparse_bt=f_sbt, sparse_ctx=f_sctx, out=f_out)
    torch.cuda.synchronize()
    assert torch.equal(f_topk, topk) and torch.equal(f_sbt, sbt) and torch.equal(f_sctx, sctx)
    assert torch.equal(f_out.view(torch.int16), out.view(torch.int16))
    assert f_out.shape == (T, cfg.num_q_heads, 128) and sbt.shape[0] == T * H_kv


# ------------------------------------------------------------------ attention
def _synthetic_table(hi, seed):
    cfg = hi["cfg"]
    rng = np.random.default_rng(seed)
    T = cfg.num_tokens
    s = rng.standard_normal((cfg.num_kv_heads, T, cfg.max_blocks))
    topk = od.topk_select(s, hi["seq_lens"], cfg.query_len, cfg.top_k)
    return od.emit_sparse_block_table(topk, hi["block_table"], hi["seq_lens"], cfg.query_len,
                                      cfg.num_kv_heads, cfg.top_k, cfg.pages_per_block)


@pytest.mark.parametrize("name", list(SMALL))
def test_sparse_pa_parity(name):
    _say(f"[sparse_pa] {name}")
    w, layer, hi = _run_small(name)
    cfg = w.cfg
    sbt, sctx = _synthetic_table(hi, 5)
    ref = oracle_attention(hi, sbt, sctx)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               torch.from_numpy(sbt).cuda(), torch.from_numpy(sctx).cuda(),
                               cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale,
                               decode_query_len=cfg.query_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all(), "NaN in attention output (poison read?)"
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hi, sbt, sctx))
    err = np.abs(got - ref).max()
    assert err <= tol, f"max |err| {err:.4g} > {tol:.4g}"
    empty = np.nonzero(sctx.reshape(cfg.num_tokens, cfg.num_kv_heads).sum(axis=1) == 0)[0]
    assert (got[empty] == 0).all()


# Query / cache dtype pairs and head groupings the five workloads do not use,
# and rows with more splits than the merging workgroup loads at once.
_PA_VARIANTS = {
    "mxfp4_kv_bf16_q": ("mxfp4", dict(q_dtype="bf16")),
    "bf16_kv_e4m3_q": ("tiny_bf16", dict(q_dtype="e4m3")),
    "fp8_kv_e4m3_q": ("fp8_decode", dict(q_dtype="e4m3")),
    "fp8_two_kv_heads": ("fp8_decode", dict(num_kv_heads=2, num_q_heads=16)),
    "mxfp4_two_kv_heads": ("mxfp4", dict(num_kv_heads=2, num_q_heads=16)),
    "fp8_group_of_4": ("fp8_decode", dict(num_q_heads=4)),
    "fp8_18_splits": ("fp8_decode", dict(top_k=72)),
    "mxfp4_10_splits": ("mxfp4", dict(top_k=40)),
}


@pytest.mark.parametrize("base", ["spec_decode", "tiny_bf16"])
def test_sparse_pa_one_split_several_rounds(base):
    # Enough rows to fill the chip: one split a row, walked in several rounds
    # with the running max carried between them (fp8 runs of 8 pages, bf16 of 4).
    reqs = 150 if base == "spec_decode" else 520   # >= 512 rows either way
    cfg = wl.shrink(wl.CONFIGS[base], num_reqs=reqs, ctx_lo=1500, ctx_hi=3000, num_pad_reqs=3,
                    pool_blocks=reqs * 24 + 64, top_k=12)
    _say(f"[sparse_pa rounds] {base}: {cfg.num_tokens} rows")
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    sbt, sctx = _synthetic_table(hi, 21)
    rows = cfg.num_tokens * cfg.num_kv_heads
    assert rows >= 512 and sbt.shape[1] > 4 * (8 if cfg.kv_dtype == "fp8" else 4)
    ref = oracle_attention(hi, sbt, sctx)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               torch.from_numpy(sbt).cuda(), torch.from_numpy(sctx).cuda(),
                               cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale,
                               decode_query_len=cfg.query_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hi, sbt, sctx))
    err = np.abs(got - ref).max()
    assert err <= tol, f"max |err| {err:.4g} > {tol:.4g}"


@pytest.mark.parametrize("variant", list(_PA_VARIANTS))
def test_sparse_pa_variants(variant):
    base, kw = _PA_VARIANTS[variant]
    cfg = dataclasses.replace(SMALL[base], **kw)
    if "splits" in variant:
        cfg = dataclasses.replace(wl.shrink(SMALL[base], num_reqs=3, ctx_lo=9000, ctx_hi=12000), **kw)
    _say(f"[sparse_pa variant] {variant}: {cfg}")
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    sbt, sctx = _synthetic_table(hi, 11)
    ref = oracle_attention(hi, sbt, sctx)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               torch.from_numpy(sbt).cuda(), torch.from_numpy(sctx).cuda(),
                               cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale,
                               decode_query_len=cfg.query_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all(), "NaN in attention output (poison read?)"
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hi, sbt, sctx))
    err = np.abs(got - ref).max()
    assert err <= tol, f"max |err| {err:.4g} > {tol:.4g}"


# Any row count: the split plan gives small batches many splits a row (every
# page in flight at once) and large ones a single split; the counts cross the
# plan's steps (512 resident four-wave workgroups) and leave ragged final
# rounds.  (128, 16) and (150, 12) take two splits of eight-wave workgroups,
# (256, 8) one split of eight waves.
@pytest.mark.parametrize("reqs,top_k", [(1, 8), (2, 8), (5, 8), (33, 8), (129, 8), (257, 8), (511, 8), (700, 8),
                                        (128, 16), (150, 12), (256, 8),
                                        (1984, 8), (2049, 4)])   # one wave a row from 1984 rows
def test_sparse_pa_row_counts(reqs, top_k):
    cfg = wl.shrink(wl.CONFIGS["fp8_decode"], num_reqs=reqs, ctx_lo=200, ctx_hi=5000,
                    pool_blocks=reqs * 40 + 64, top_k=top_k)
    _say(f"[sparse_pa rows] {reqs} rows, top-k {top_k}")
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    sbt, sctx = _synthetic_table(hi, 31 + reqs)
    ref = oracle_attention(hi, sbt, sctx)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               torch.from_numpy(sbt).cuda(), torch.from_numpy(sctx).cuda(),
                               cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale,
                               decode_query_len=cfg.query_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all(), "NaN in attention output (poison read?)"
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hi, sbt, sctx))
    err = np.abs(got - ref).max()
    assert err <= tol, f"max |err| {err:.4g} > {tol:.4g}"


@pytest.mark.parametrize("base,kw", [("tiny_bf16", dict(num_q_heads=16)),
                                     ("fp8_decode", dict(num_kv_heads=2, num_q_heads=16, num_idx_heads=2)),
                                     ("fp8_decode", dict(q_dtype="e4m3"))])
def test_sparse_pa_one_wave_a_row(base, kw):
    # batches of at least 1984 rows of 16-token pages give every row a wave of
    # its own: bf16 pages, two KV heads (row = token, head), an e4m3 query
    reqs = 1000 if kw.get("num_kv_heads") == 2 else 2000
    cfg = wl.shrink(dataclasses.replace(wl.CONFIGS[base], **kw), num_reqs=reqs, ctx_lo=100, ctx_hi=1500,
                    pool_blocks=reqs * 13 + 64, top_k=6)
    _say(f"[sparse_pa one wave a row] {base} {kw}")
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    sbt, sctx = _synthetic_table(hi, 77)
    ref = oracle_attention(hi, sbt, sctx)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               torch.from_numpy(sbt).cuda(), torch.from_numpy(sctx).cuda(),
                               cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale, decode_query_len=cfg.query_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hi, sbt, sctx))
    err = np.abs(got - ref).max(axis=(1, 2))
    assert (err <= tol).all(), f"max |err| {err.max():.4g} > {tol:.4g}"


def test_sparse_pa_one_wave_a_row_long_rows_and_empty_rows():
    # one wave a row with sixteen runs a row (the page ids of runs 8.. are
    # fetched mid-walk) and rows of length 0 among them
    cfg = wl.shrink(wl.CONFIGS["fp8_decode"], num_reqs=2000, ctx_lo=100, ctx_hi=2500, num_pad_reqs=40,
                    pool_blocks=2040 * 20 + 64, top_k=16)
    _say("[sparse_pa one wave a row] sixteen runs, empty rows")
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    sbt, sctx = _synthetic_table(hi, 78)
    assert (sctx == 0).sum() >= 40 and sbt.shape[1] == 128
    ref = oracle_attention(hi, sbt, sctx)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               torch.from_numpy(sbt).cuda(), torch.from_numpy(sctx).cuda(),
                               cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale, decode_query_len=cfg.query_len)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    assert (got[sctx == 0] == 0).all()
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hi, sbt, sctx))
    err = np.abs(got - ref).max(axis=(1, 2))
    assert (err <= tol).all(), f"max |err| {err.max():.4g} > {tol:.4g}"


def test_sparse_pa_every_block_is_dense_attention():
    # top-k >= every row's block count: the sparse decode is dense causal attention.
    cfg = wl.shrink(wl.CONFIGS["fp8_decode"], num_reqs=4, ctx_lo=100, ctx_hi=2000, top_k=16)
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    topk = od.topk_select(np.zeros((1, cfg.num_tokens, cfg.max_blocks)), hi["seq_lens"], 1, 16)
    assert (topk[0, :, :] >= 0).sum() == sum(-(-int(L) // 128) for L in hi["seq_lens"])
    sbt, sctx = od.emit_sparse_block_table(topk, hi["block_table"], hi["seq_lens"], 1, 1, 16, 8)
    assert list(sctx) == list(hi["seq_lens"])
    ref = oracle_attention(hi, sbt, sctx)
    out = isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                               torch.from_numpy(sbt).cuda(), torch.from_numpy(sctx).cuda(), 16, 1, w.sm_scale,
                               decode_query_len=cfg.query_len)
    torch.cuda.synchronize()
    tol = attn_tol("fp8", attended_vmax(hi, sbt, sctx))
    assert np.abs(out.float().cpu().numpy() - ref).max() <= tol


def test_sparse_pa_repeat_calls_and_output_contents():
    # The output's prior contents do not matter: three calls with differently
    # filled outputs give bit-identical results, and each call leaves the
    # workspace as it found it (zero: every split slot free).
    for name in ("long_context", "fp8_decode", "mxfp4"):
        w, layer, hi = _run_small(name)
        cfg = w.cfg
        outs = []
        ws = isb.binding.new_workspace(layer.workspace.numel(), "cuda")
        for fill in (float("nan"), 0.0, float("inf")):
            out = torch.full((cfg.num_tokens, cfg.num_q_heads, 128), fill, dtype=torch.bfloat16, device="cuda")
            isb.sparse_pa_decode(w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale,
                                 layer.sparse_bt, layer.sparse_ctx, cfg.num_q_heads, cfg.num_kv_heads,
                                 w.sm_scale, out=out, workspace=ws, decode_query_len=cfg.query_len)
            outs.append(out)
            torch.cuda.synchronize()
            assert not bool(ws.any()), "a split slot was left occupied"
        for o in outs[1:]:
            assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))
        assert torch.equal(outs[0].view(torch.int16), layer.out.view(torch.int16))


# ------------------------------------------------------------------ chained layer
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_chain(name):
    _say(f"[chain] {name}")
    w, layer, hi = _run_small(name)
    ref = oracle_layer(hi)
    check_chain(hi, layer.scores.cpu().numpy().astype(np.float64), layer.topk.cpu().numpy(),
                 layer.sparse_bt.cpu().numpy(), layer.sparse_ctx.cpu().numpy(),
                 layer.out.float().cpu().numpy(), ref, hi["block_table"])


# ------------------------------------------------------------------ graph capture
@pytest.mark.parametrize("name", ["fp8_decode", "spec_decode", "mxfp4"])
def test_layer_replays_from_a_hip_graph(name):
    # The calls allocate nothing and never synchronise, so a layer step can be
    # captured; every replay (with eager work and syncs in between) must give
    # the eager step's outputs bit for bit, and leave every workspace slot
    # free for the next call.
    _say(f"[graph] {name}")
    w = wl.make_workload(SMALL[name], device="cuda")
    layer = isb.DecodeLayer(w)
    layer.run()
    torch.cuda.synchronize()
    want = [t.clone() for t in (layer.scores, layer.topk, layer.sparse_bt, layer.sparse_ctx, layer.out)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up on the capturing stream
        layer.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.run()
    rows = w.cfg.num_tokens * w.cfg.num_kv_heads
    for rep in range(4):
        for t in (layer.scores, layer.out):
            t.fill_(float("nan"))            # eager work between replays
        layer.topk.fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (layer.scores, layer.topk, layer.sparse_bt, layer.sparse_ctx, layer.out)
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               b.view(torch.uint8) if b.dtype != torch.int32 else b), f"replay {rep}"
        assert not bool(layer.workspace.any()), f"replay {rep}: a split slot was left occupied"


# ------------------------------------------------------------------ full size, sampled
FULL_SAMPLES = {"tiny_bf16": [0, 1, 2, 3], "fp8_decode": [3, 77], "spec_decode": None,
                "mxfp4": [5, 60], "long_context": [6], "prefill": [2], "prefill_e4m3q": [1]}


@pytest.mark.parametrize("name", list(FULL_SAMPLES))
def test_full_size_sampled(name):
    cfg = wl.CONFIGS[name]
    _say(f"[full] {name}: generating")
    w = wl.make_workload(cfg, device="cuda")
    layer = isb.DecodeLayer(w)
    layer.run()
    torch.cuda.synchronize()
    reqs = FULL_SAMPLES[name]
    if reqs is None:  # two live requests and one pad request
        lens = w.seq_lens.cpu().numpy()
        reqs = [int(np.nonzero(lens > 0)[0][0]), int(np.nonzero(lens > 0)[0][-1]), int(np.nonzero(lens == 0)[0][0])]
    _say(f"[full] {name}: oracle on requests {reqs}")
    hi, toks, remap = sample_requests(w, reqs)
    ref = oracle_layer(hi)
    H_kv = cfg.num_kv_heads
    rows = [t * H_kv + g for t in toks for g in range(H_kv)]
    bt_global = w.block_table[reqs].cpu().numpy()
    check_chain(hi, layer.scores[:, toks, :].cpu().numpy().astype(np.float64),
                 layer.topk[:, toks, :].cpu().numpy(), layer.sparse_bt[rows].cpu().numpy(),
                 layer.sparse_ctx[rows].cpu().numpy(), layer.out[toks].float().cpu().numpy(), ref,
                 bt_global, remap)
    del w, layer
    torch.cuda.empty_cache()
