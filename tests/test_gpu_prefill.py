"""GPU parity of the prefill calls: ragged batches where every token has its
own request id and position (needs an MI355X).

* Mixed chunk lengths in one call (a single token up to several query tiles,
  requests with no tokens), tokens grouped by request or shuffled, one or two
  KV heads, one or four index heads, fp8 / bf16 / MXFP4 caches: the chained
  layer against the prefill oracle on every row, as for decode (scores within
  1e-3 relative; the oracle's top-k of the GPU's own fp32 scores and its emit
  of the GPU's selection bit-exact; the oracle's attention over the GPU's
  table within the attention tolerance).
* Each call on its own (scorer, top-k, emit, top-k + emit, attention, select
  + attend) against the oracle or against the other calls, bit for bit.
* Shuffling the tokens permutes every output bit for bit.
* Tokens with a request id or position out of range are empty rows.
* The full-size ragged batch in the launch configuration the benchmark
  times, on sampled tokens.
"""
import numpy as np
import pytest
import torch

import indexer_selected_block_amd as isb
from indexer_selected_block_amd import workload as wl
from oracle import formats
from oracle import prefill as op

from _util import assert_scores_close, attended_vmax, attn_tol, oracle_attention, selection_margin_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    isb.load_library()


def _say(*a):
    print(*a, flush=True)


def _cfg(base, R, lo, hi, **kw):
    c = wl.ragged_config(base) if base in wl.RAGGED_CHUNKS else wl.CONFIGS[base]
    return wl.shrink(wl.replace(c, **kw) if kw else c, num_reqs=R, ctx_lo=lo, ctx_hi=hi, num_pad_reqs=0)


# name -> (config, chunk lengths, token order)
CASES = {
    "fp8_mixed": (_cfg("prefill_ragged", 6, 600, 3000), (150, 1, 37, 0, 200, 9), "grouped"),
    "fp8_shuffled": (_cfg("prefill_ragged", 6, 600, 3000), (150, 1, 37, 0, 200, 9), "shuffled"),
    "mxfp4_four_index_heads": (_cfg("mxfp4", 3, 900, 2500), (40, 3, 70), "grouped"),
    "bf16": (_cfg("tiny_bf16", 4, 300, 1024), (70, 5, 1, 30), "grouped"),
    "two_kv_heads": (_cfg("prefill_ragged", 3, 500, 2500, num_kv_heads=2, num_idx_heads=2),
                     (33, 64, 17), "shuffled"),
}

_cache = {}


def _host(w, b):
    h = w.to("cpu")
    cfg = h.cfg
    bh = b.to("cpu")
    return dict(cfg=cfg, block_table=h.block_table.numpy(), req=bh.query_req_id.numpy(),
                pos=bh.query_abs_pos.numpy(), q=formats.decode_query(bh.q.numpy(), cfg.q_dtype),
                q_idx=formats.decode_query(bh.q_idx.numpy(), cfg.qidx_dtype), idx_pool=h.idx_pool.numpy(),
                k_pool=h.k_pool.numpy(), v_pool=h.v_pool.numpy(), idx_scale=h.idx_scale, k_scale=h.k_scale,
                v_scale=h.v_scale, sm_scale=h.sm_scale)


def _oracle(hp):
    cfg = hp["cfg"]
    return op.prefill_layer(hp["q"], hp["q_idx"], hp["idx_pool"], cfg.idx_dtype, hp["idx_scale"], hp["k_pool"],
                            hp["v_pool"], cfg.kv_dtype, hp["k_scale"], hp["v_scale"], hp["block_table"],
                            hp["req"], hp["pos"], cfg.num_kv_heads, cfg.max_blocks, cfg.top_k,
                            cfg.pages_per_block, hp["sm_scale"])


def _run(name):
    if name not in _cache:
        cfg, chunks, order = CASES[name]
        w = wl.make_workload(cfg, device="cuda")
        b = wl.ragged_batch(w, chunks, order=order, seed=1)
        layer = isb.PrefillLayer(w, b)
        layer.run()
        torch.cuda.synchronize()
        hp = _host(w, b)
        _cache[name] = (w, b, layer, hp, _oracle(hp))
    return _cache[name]


def check_prefill_chain(hp, scores, topk, sbt, sctx, out, ref):
    """The GPU's prefill layer against the oracle fed the GPU's own results,
    every row (see the decode chain check)."""
    cfg = hp["cfg"]
    H_kv, K, ppb = cfg.num_kv_heads, cfg.top_k, cfg.pages_per_block
    scores32 = np.asarray(scores, dtype=np.float32)
    assert_scores_close(scores32, ref["scores"])
    topk_ref = op.topk_select_prefill(scores32, hp["pos"], K)
    diff = np.nonzero(~np.all(topk_ref == topk, axis=-1))
    assert diff[0].size == 0, f"{diff[0].size} rows select differently from the oracle on the same scores"
    with np.errstate(invalid="ignore"):
        err_row = np.where(np.isfinite(ref["scores"]), np.abs(scores32 - ref["scores"]), 0).max(axis=-1)
    for g in range(H_kv):
        for t in range(topk.shape[1]):
            if not np.array_equal(topk[g, t], ref["topk"][g, t]):
                nt = -(-(int(hp["pos"][t]) + 1) // 128)
                assert selection_margin_ok(ref["scores"][g, t], nt, K, list(topk[g, t]), 2 * err_row[g, t] + 1e-12)
    sbt_ref, sctx_ref = op.emit_sparse_block_table_prefill(topk, hp["block_table"], hp["req"], hp["pos"], H_kv, K,
                                                           ppb)
    assert np.array_equal(sbt, sbt_ref), "sparse page table differs"
    assert np.array_equal(sctx, sctx_ref), "sparse lengths differ"
    out_ref = oracle_attention(hp, sbt, sctx)
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hp, sbt, sctx))
    assert np.isfinite(out).all(), "NaN in the attention output"
    err = np.abs(out - out_ref).max(axis=(1, 2))
    assert (err <= tol).all(), f"attention err {err.max():.4g} > {tol:.4g} on {(err > tol).sum()} tokens"


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_layer_chain(name):
    _say(f"[prefill chain] {name}")
    w, b, layer, hp, ref = _run(name)
    check_prefill_chain(hp, layer.scores.cpu().numpy(), layer.topk.cpu().numpy(), layer.sparse_bt.cpu().numpy(),
                        layer.sparse_ctx.cpu().numpy(), layer.out.float().cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["fp8_mixed", "mxfp4_four_index_heads", "two_kv_heads"])
def test_prefill_calls_one_by_one(name):
    """top-k, emit, top-k + emit and attention each on its own: the oracle's
    top-k and emit bit for bit; the attention call equal to select + attend's."""
    _say(f"[prefill calls] {name}")
    w, b, layer, hp, ref = _run(name)
    cfg = w.cfg
    scores = layer.scores
    topk = isb.topk_select_prefill(scores, w.block_table.shape[0], b.query_req_id, b.query_abs_pos, cfg.top_k)
    assert torch.equal(topk, layer.topk)
    np.testing.assert_array_equal(topk.cpu().numpy(),
                                  op.topk_select_prefill(scores.cpu().numpy(), hp["pos"], cfg.top_k))
    sbt, sctx = isb.emit_sparse_block_table_prefill(topk, w.block_table, b.query_req_id, b.query_abs_pos,
                                                    cfg.pages_per_block)
    assert torch.equal(sbt, layer.sparse_bt) and torch.equal(sctx, layer.sparse_ctx)
    t2, s2, c2 = isb.topk_select_emit_prefill(scores, b.query_req_id, b.query_abs_pos, cfg.top_k, w.block_table,
                                              cfg.pages_per_block)
    assert torch.equal(t2, topk) and torch.equal(s2, sbt) and torch.equal(c2, sctx)
    out = isb.sparse_pa_prefill(b.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, sbt, sctx,
                                cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), layer.out.view(torch.int16))


def test_shuffled_tokens_permute_every_output():
    """The same tokens in another order: every output permuted, bit for bit."""
    w, b, layer, _, _ = _run("fp8_mixed")
    perm = torch.randperm(b.num_tokens, generator=torch.Generator().manual_seed(9)).cuda()
    bs = wl.RaggedBatch(b.query_req_id[perm].contiguous(), b.query_abs_pos[perm].contiguous(),
                        b.q[perm].contiguous(), b.q_idx[perm].contiguous())
    other = isb.PrefillLayer(w, bs)
    other.run()
    torch.cuda.synchronize()
    assert torch.equal(other.scores, layer.scores[:, perm])
    assert torch.equal(other.topk, layer.topk[:, perm])
    assert torch.equal(other.sparse_bt, layer.sparse_bt[perm])      # one KV head: row = token
    assert torch.equal(other.sparse_ctx, layer.sparse_ctx[perm])
    assert torch.equal(other.out.view(torch.int16), layer.out[perm].view(torch.int16))


def test_out_of_range_tokens_are_empty_rows():
    """Request ids outside [0, num_reqs) and positions outside [0, 128
    max_blocks) give -inf scores, no selection, length 0 and zero output; the
    valid tokens of the same call are unaffected."""
    w, b, layer, _, _ = _run("fp8_mixed")
    cfg = w.cfg
    R, MB = w.block_table.shape[0], cfg.max_blocks
    bad_req = torch.tensor([-1, R, 0, 2, 1 << 30], dtype=torch.int32)
    bad_pos = torch.tensor([5, 5, -3, 128 * MB, 7], dtype=torch.int32)
    n = b.num_tokens
    where = torch.tensor([0, 3, n // 2, n // 2 + 1, n + 4])           # slots in the longer batch
    keep = torch.ones(n + 5, dtype=torch.bool)
    keep[where] = False
    req = torch.empty(n + 5, dtype=torch.int32)
    pos = torch.empty(n + 5, dtype=torch.int32)
    req[keep], pos[keep] = b.query_req_id.cpu(), b.query_abs_pos.cpu()
    req[where], pos[where] = bad_req, bad_pos
    q = torch.zeros((n + 5,) + tuple(b.q.shape[1:]), dtype=b.q.dtype)
    qi = torch.zeros((n + 5,) + tuple(b.q_idx.shape[1:]), dtype=b.q_idx.dtype)
    q[keep], qi[keep] = b.q.cpu(), b.q_idx.cpu()
    bb = wl.RaggedBatch(req.cuda(), pos.cuda(), q.cuda(), qi.cuda())
    big = isb.PrefillLayer(w, bb)
    big.run()
    torch.cuda.synchronize()
    kd, wd = keep.cuda(), where.cuda()
    assert torch.equal(big.scores[:, kd], layer.scores)
    assert torch.equal(big.topk[:, kd], layer.topk)
    assert torch.equal(big.sparse_bt[kd], layer.sparse_bt) and torch.equal(big.sparse_ctx[kd], layer.sparse_ctx)
    assert torch.equal(big.out[kd].view(torch.int16), layer.out.view(torch.int16))
    assert bool(torch.isneginf(big.scores[:, wd]).all())
    assert bool((big.topk[:, wd] == -1).all()) and bool((big.sparse_bt[wd] == -1).all())
    assert bool((big.sparse_ctx[wd] == 0).all())
    assert bool((big.out[wd].float() == 0).all())


def test_prefill_replays_from_a_hip_graph():
    """A captured prefill step replays the eager outputs bit for bit."""
    w, b, layer, _, _ = _run("fp8_shuffled")
    want = [t.clone() for t in (layer.scores, layer.topk, layer.sparse_bt, layer.sparse_ctx, layer.out)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.run()
    for rep in range(3):
        layer.scores.fill_(float("nan"))
        layer.out.fill_(float("nan"))
        layer.topk.fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (layer.scores, layer.topk, layer.sparse_bt, layer.sparse_ctx, layer.out)
        for a, c in zip(got, want):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               c.view(torch.uint8) if c.dtype != torch.int32 else c), f"replay {rep}"
        assert not bool(layer.workspace.any())


def test_full_size_ragged_prefill_sampled():
    """The whole ragged batch (six requests, chunks of 1 to 1024 tokens,
    contexts up to 65536) in the benchmark's launch configuration; the oracle
    recomputes sampled tokens of every request from the full pools."""
    name = "prefill_ragged"
    cfg = wl.ragged_config(name)
    _say(f"[full prefill] {name}: generating")
    w = wl.make_workload(cfg, device="cuda")
    b = wl.ragged_batch(w, wl.RAGGED_CHUNKS[name])
    layer = isb.PrefillLayer(w, b)
    layer.run()
    torch.cuda.synchronize()
    req = b.query_req_id.cpu().numpy()
    toks = []
    for r in range(cfg.num_reqs):
        mine = np.nonzero(req == r)[0]
        if mine.size:
            toks += sorted({int(mine[0]), int(mine[-1]), int(mine[mine.size // 2])})
    _say(f"[full prefill] {name}: oracle on tokens {toks}")
    sub = wl.RaggedBatch(*(t[toks] for t in (b.query_req_id, b.query_abs_pos, b.q, b.q_idx)))
    hp = _host(w, sub)
    ref = _oracle(hp)
    H_kv = cfg.num_kv_heads
    rows = [t * H_kv + g for t in toks for g in range(H_kv)]
    check_prefill_chain(hp, layer.scores[:, toks].cpu().numpy(), layer.topk[:, toks].cpu().numpy(),
                        layer.sparse_bt[rows].cpu().numpy(), layer.sparse_ctx[rows].cpu().numpy(),
                        layer.out[toks].float().cpu().numpy(), ref)
    del w, layer
    torch.cuda.empty_cache()
