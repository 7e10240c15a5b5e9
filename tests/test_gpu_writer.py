"""GPU parity of the cache writer and the e4m3 query cast against the oracle.

Both sides start from the same pool bytes and the same bf16 new tokens; the
pools the GPU writes must equal the oracle's byte for byte (integer work:
bit-exact), including the pages no token touches.  The inputs mix normal
values with the encodings' edge cases: ties between adjacent codes, values
past the saturation points, subnormal e4m3 values, signed zeros, all-zero MX
groups and NaN (fp8 only).  Full-size cases write one step of new tokens into
the decode workloads' own pools and compare the touched pages against the
oracle run on those pages alone, then check that no other byte changed.
"""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import indexer_selected_block_amd as isb
from indexer_selected_block_amd import workload as wl
from oracle import formats, writer

pytestmark = pytest.mark.gpu

KV_PAGE = {"bf16": 4096, "fp8": 2048, "mxfp4": formats.MXFP4_PAGE_BYTES}
IDX_PAGE = {"bf16": 32768, "fp8": 16384, "mxfp4": formats.MXFP4_PAGE_BYTES}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    isb.load_library()


def _say(*a):
    print(*a, flush=True)


def _edge_values(rng, n, dtype):
    """n bf16 values: normals at mixed magnitudes plus the encodings' edge cases."""
    x = rng.standard_normal(n) * np.exp2(rng.integers(-6, 6, n))
    e4m3 = np.array([formats.e4m3_value(c) for c in range(0x7F)])
    specials = np.concatenate([
        (e4m3[:-1] + e4m3[1:]) / 2,                  # e4m3 ties (exact in bf16)
        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0],     # e2m1 ties at a group scale of 1
        [448.0, 464.0, 1e4, 2.0 ** -10, 2.0 ** -9 * 3, -0.0, 0.0]])
    k = min(len(specials), n // 2)
    pos = rng.choice(n, size=k, replace=False)
    x[pos] = rng.permutation(specials)[:k] * rng.choice([-1, 1], k)
    if dtype == "fp8" and n >= 8:
        x[rng.choice(n, size=2, replace=False)] = np.nan
    return x


# An MX group whose maximum 4 gives it the exponent 0, holding every e2m1 tie
# (then scaled by 2^s: the same ties at the exponent s).
_MX_TIES = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4) * np.tile([1, 1, 1, 1, -1, -1, -1, -1], 4)


def _new_tokens(rng, T, H_kv, kv_dtype, idx_dtype):
    def bf16(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)

    k = bf16(_edge_values(rng, T * H_kv * 128, kv_dtype).reshape(T, H_kv, 128))
    v = bf16(_edge_values(rng, T * H_kv * 128, kv_dtype).reshape(T, H_kv, 128))
    i = bf16(_edge_values(rng, T * 128, idx_dtype).reshape(T, 128))
    if kv_dtype == "mxfp4" and T:
        k[0, 0, :32] = 0                                     # an all-zero MX group
        k[0, 0, 32:64] = torch.from_numpy(_MX_TIES).to(torch.bfloat16)
        v[-1, -1, 96:] = torch.from_numpy(_MX_TIES * 2.0 ** -20).to(torch.bfloat16)
    if idx_dtype == "mxfp4" and T:
        i[0, 64:96] = torch.from_numpy(_MX_TIES * 2.0 ** -3).to(torch.bfloat16)
    return k, v, i


def _host(t):
    return t.float().double().numpy()


CASES = {
    # name: (kv dtype, index dtype, H_kv, query_len, seq_lens, table width, pool blocks)
    "fp8_fp8_decode": ("fp8", "fp8", 1, 1, [300, 1, 0, 4097, 128], 40, 64),
    "fp8_fp8_spec_h2": ("fp8", "fp8", 2, 4, [300, 2, 0, 4097, 129, 3], 40, 64),
    "bf16_bf16": ("bf16", "bf16", 2, 3, [300, 2, 0, 1000], 10, 48),
    "mxfp4_mxfp4": ("mxfp4", "mxfp4", 1, 4, [300, 2, 0, 4097, 129], 40, 64),
    "mxfp4_mxfp4_h2": ("mxfp4", "mxfp4", 2, 3, [260, 2, 0, 900], 10, 48),
    "fp8_kv_mxfp4_idx": ("fp8", "mxfp4", 1, 2, [300, 1, 0, 513], 8, 40),
    "bf16_kv_fp8_idx": ("bf16", "fp8", 1, 5, [640, 4, 0, 700], 8, 40),
    "mxfp4_kv_bf16_idx": ("mxfp4", "bf16", 2, 2, [130, 1, 0, 257], 8, 40),
    "prefill_chunk": ("fp8", "fp8", 1, 150, [600, 149, 0, 2000], 16, 48),
}


def _case_inputs(name):
    kv, idt, H, q, lens, width, nblk = CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    R = len(lens)
    # each request's blocks distinct from every other's (no two tokens share a
    # slot); table entries past a request's blocks hold arbitrary ids
    bt = rng.integers(0, nblk, (R, width)).astype(np.int32)
    need = [-(-L // 128) for L in lens]
    assert sum(need) <= nblk and max(need) <= width
    ids = rng.permutation(nblk)
    for r in range(R):
        bt[r, :need[r]] = ids[sum(need[:r]):sum(need[:r + 1])]
    npages = nblk * (8 if kv != "mxfp4" else 1)
    pools = dict(k=rng.integers(0, 256, (npages, H * KV_PAGE[kv]), dtype=np.uint8),
                 v=rng.integers(0, 256, (npages, H * KV_PAGE[kv]), dtype=np.uint8),
                 i=rng.integers(0, 256, (nblk, IDX_PAGE[idt]), dtype=np.uint8))
    k_new, v_new, i_new = _new_tokens(rng, R * q, H, kv, idt)
    return kv, idt, H, q, np.array(lens, np.int32), bt, pools, (k_new, v_new, i_new)


def _gpu_write(kv, idt, q, lens, bt, pools, news, ks, vs, xs, with_idx=True):
    dev = "cuda"
    d = {n: torch.from_numpy(a).to(dev) for n, a in pools.items()}
    k_new, v_new, i_new = (t.to(dev) for t in news)
    isb.write_cache(k_new, v_new, i_new if with_idx else None, torch.from_numpy(bt).to(dev),
                    torch.from_numpy(lens).to(dev), q, d["k"], d["v"], kv, ks, vs,
                    d["i"] if with_idx else None, idt, xs)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in d.items()}


@pytest.mark.parametrize("name", list(CASES))
def test_write_cache_bit_exact(name):
    kv, idt, H, q, lens, bt, pools, news = _case_inputs(name)
    # unit scales in the decode case: the e4m3 ties among the inputs stay ties
    ks, vs, xs = (1.0, 1.0, 1.0) if name.endswith("decode") else (0.013, 0.021, 0.037)
    _say(f"write_cache {name}: kv {kv} idx {idt} H_kv {H} q {q} lens {lens.tolist()}")
    got = _gpu_write(kv, idt, q, lens, bt, pools, news, ks, vs, xs)
    ref = {n: a.copy() for n, a in pools.items()}
    writer.write_cache(_host(news[0]), _host(news[1]), _host(news[2]), bt, lens, q, ref["k"], ref["v"], kv,
                       ks, vs, ref["i"], idt, xs)
    for n in ("k", "v", "i"):
        bad = np.argwhere(got[n] != ref[n])
        assert bad.size == 0, f"pool {n}: {len(bad)} bytes differ, first at {bad[:4].tolist()}"
    assert any(not np.array_equal(got[n], pools[n]) for n in ("k", "v", "i"))


@pytest.mark.parametrize("name", ["fp8_fp8_spec_h2", "mxfp4_mxfp4"])
def test_write_cache_without_index_key(name):
    kv, idt, H, q, lens, bt, pools, news = _case_inputs(name)
    _say(f"write_cache (no index key) {name}")
    got = _gpu_write(kv, idt, q, lens, bt, pools, news, 0.02, 0.03, 0.05, with_idx=False)
    ref = {n: a.copy() for n, a in pools.items()}
    writer.write_cache(_host(news[0]), _host(news[1]), None, bt, lens, q, ref["k"], ref["v"], kv, 0.02, 0.03,
                       ref["i"], idt, 0.05)
    for n in ("k", "v", "i"):
        assert np.array_equal(got[n], ref[n]), n
    assert np.array_equal(got["i"], pools["i"])


def test_write_cache_skips_blocks_outside_the_pools():
    # a table row whose ids fall outside the pools writes nothing; the rest is
    # written as if that request were a pad request
    kv, idt, H, q, lens, bt, pools, news = _case_inputs("fp8_fp8_spec_h2")
    bt_bad = bt.copy()
    bt_bad[3] = 64 + np.arange(bt.shape[1])                  # 64 blocks in the pools
    bt_bad[0, 2] = -1                                        # request 0 writes at positions 296..299
    _say("write_cache out-of-pool ids")
    got = _gpu_write(kv, idt, q, lens, bt_bad, pools, news, 0.02, 0.03, 0.05)
    lens_ref = lens.copy()
    lens_ref[[0, 3]] = 0
    ref = {n: a.copy() for n, a in pools.items()}
    writer.write_cache(_host(news[0]), _host(news[1]), _host(news[2]), bt, lens_ref, q, ref["k"], ref["v"], kv,
                       0.02, 0.03, ref["i"], idt, 0.05)
    for n in ("k", "v", "i"):
        assert np.array_equal(got[n], ref[n]), n


# The writer of the decode workloads at their full sizes: one step of new
# tokens, every request's tokens written into the workload's own pools.
FULL = ["fp8_decode", "spec_decode", "mxfp4"]


@pytest.mark.parametrize("name", FULL)
def test_write_cache_full_size(name):
    cfg = wl.CONFIGS[name]
    w = wl.make_workload(cfg, device="cuda")
    rng = np.random.default_rng(11)
    T, H, q = cfg.num_tokens, cfg.num_kv_heads, cfg.query_len
    news = _new_tokens(rng, T, H, cfg.kv_dtype, cfg.idx_dtype)
    lens = w.seq_lens.cpu().numpy()
    bt = w.block_table.cpu().numpy()
    blocks = sorted({int(bt[r, p // 128]) for r in range(len(lens))
                     for p in range(max(0, int(lens[r]) - q), int(lens[r]))})
    _say(f"write_cache full {name}: T {T} blocks touched {len(blocks)}")
    ppb = 1 if cfg.kv_dtype == "mxfp4" else 8
    kv_rows = torch.tensor([ppb * b + j for b in blocks for j in range(ppb)], device="cuda")
    ix_rows = torch.tensor(blocks, device="cuda")
    before = dict(k=w.k_pool.clone(), v=w.v_pool.clone(), i=w.idx_pool.clone())
    isb.write_cache(*(t.cuda() for t in news), w.block_table, w.seq_lens, q, w.k_pool, w.v_pool, cfg.kv_dtype,
                    w.k_scale, w.v_scale, w.idx_pool, cfg.idx_dtype, w.idx_scale)
    torch.cuda.synchronize()
    # the oracle on the touched pages alone, block ids renumbered 0..n-1
    remap = np.full(int(bt.max()) + 1, -1, np.int64)
    remap[blocks] = np.arange(len(blocks))
    bt_c = np.where(bt >= 0, remap[np.clip(bt, 0, None)], -1)
    ref = dict(k=before["k"][kv_rows].cpu().numpy(), v=before["v"][kv_rows].cpu().numpy(),
               i=before["i"][ix_rows].cpu().numpy())
    writer.write_cache(_host(news[0]), _host(news[1]), _host(news[2]), bt_c, lens, q, ref["k"], ref["v"],
                       cfg.kv_dtype, w.k_scale, w.v_scale, ref["i"], cfg.idx_dtype, w.idx_scale)
    got = dict(k=w.k_pool[kv_rows].cpu().numpy(), v=w.v_pool[kv_rows].cpu().numpy(),
               i=w.idx_pool[ix_rows].cpu().numpy())
    for n in ("k", "v", "i"):
        assert np.array_equal(got[n], ref[n]), n
    # every other byte of the pools is unchanged
    before["k"][kv_rows] = w.k_pool[kv_rows]
    before["v"][kv_rows] = w.v_pool[kv_rows]
    before["i"][ix_rows] = w.idx_pool[ix_rows]
    assert torch.equal(before["k"], w.k_pool) and torch.equal(before["v"], w.v_pool)
    assert torch.equal(before["i"], w.idx_pool)


@pytest.mark.parametrize("n", [1, 255, 1024, 1025, 128 * 1024 * 16 + 3])
def test_quantize_e4m3_bit_exact(n):
    rng = np.random.default_rng(n)
    x = torch.from_numpy(_edge_values(rng, n, "fp8").astype(np.float32)).to(torch.bfloat16)
    x[:1] = float("inf") if n > 4 else x[:1]
    _say(f"quantize_e4m3 n {n}")
    got = isb.quantize_e4m3(x.cuda()).cpu().numpy()
    ref = writer.quantize_query_e4m3(_host(x))
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ top-k reuse and the e4m3 index query
def test_reusing_layer_writes_kv_only_and_attends_with_the_source_selection():
    # A layer that reuses another layer's top-k: it writes its new K and V (no
    # index key) into caches of its own and attends with the source layer's
    # sparse table, with no scorer or selector of its own.  The source
    # selection comes from seeded scores, selected on both sides (the GPU's
    # bit-exact), the reusing layer's caches from the two writers.
    from _util import attended_vmax, attn_tol, host_inputs, oracle_attention, small_configs
    from oracle import decode as od

    cfg = small_configs()["spec_decode"]
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    T, H, q = cfg.num_tokens, cfg.num_kv_heads, cfg.query_len
    rng = np.random.default_rng(31)
    scores = rng.standard_normal((H, T, cfg.max_blocks)).astype(np.float32)
    _say(f"top-k reuse: {cfg.name} T {T}")
    # source layer's selection
    topk_ref = od.topk_select(scores, hi["seq_lens"], q, cfg.top_k)
    sbt_ref, sctx_ref = od.emit_sparse_block_table(topk_ref, hi["block_table"], hi["seq_lens"], q, H, cfg.top_k,
                                                   cfg.pages_per_block)
    _, sbt, sctx = isb.topk_select_emit(torch.from_numpy(scores).cuda(), w.seq_lens, q, cfg.top_k, w.block_table,
                                        cfg.pages_per_block)
    torch.cuda.synchronize()
    assert np.array_equal(sbt.cpu().numpy(), sbt_ref) and np.array_equal(sctx.cpu().numpy(), sctx_ref)
    # reusing layer: its own caches (a copy of the source's), its new tokens, its query
    k_pool, v_pool = w.k_pool.clone(), w.v_pool.clone()
    news = [torch.from_numpy(rng.standard_normal((T, H, 128)).astype(np.float32)).to(torch.bfloat16)
            for _ in range(2)]                               # finite values: the attention is compared
    isb.write_cache(news[0].cuda(), news[1].cuda(), None, w.block_table, w.seq_lens, q, k_pool, v_pool,
                    cfg.kv_dtype, w.k_scale, w.v_scale)
    qB = torch.from_numpy(rng.standard_normal((T, cfg.num_q_heads, 128)).astype(np.float32)).to(torch.bfloat16)
    out = isb.sparse_pa_decode(qB.cuda(), "bf16", k_pool, v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, sbt, sctx,
                               cfg.num_q_heads, H, w.sm_scale, decode_query_len=q)
    torch.cuda.synchronize()
    hB = dict(hi, q=_host(qB), k_pool=hi["k_pool"].copy(), v_pool=hi["v_pool"].copy())
    writer.write_cache(_host(news[0]), _host(news[1]), None, hi["block_table"], hi["seq_lens"], q, hB["k_pool"],
                       hB["v_pool"], cfg.kv_dtype, hi["k_scale"], hi["v_scale"], None, "bf16", 1.0)
    assert np.array_equal(k_pool.cpu().numpy(), hB["k_pool"]) and np.array_equal(v_pool.cpu().numpy(), hB["v_pool"])
    ref = oracle_attention(hB, sbt_ref, sctx_ref)
    got = out.float().cpu().numpy()
    tol = attn_tol(cfg.kv_dtype, attended_vmax(hB, sbt_ref, sctx_ref))
    err = np.abs(got - ref).max()
    assert err <= tol, f"max |err| {err:.4g} > {tol:.4g}"


def test_e4m3_index_query_from_the_cast_scores_like_the_oracle():
    # The e4m3 index query: a bf16 query cast by isb_quantize_e4m3, then scored
    # against the MXFP4 index cache; the oracle casts with its own encoder.
    from _util import assert_scores_close, host_inputs, small_configs
    from oracle import decode as od

    cfg = small_configs()["mxfp4"]
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    rng = np.random.default_rng(32)
    q_bf16 = torch.from_numpy((rng.standard_normal((cfg.num_tokens, cfg.num_idx_heads, 128)) * 4)
                              .astype(np.float32)).to(torch.bfloat16)
    _say(f"e4m3 index query: {cfg.name}")
    q8 = isb.quantize_e4m3(q_bf16.cuda())
    scores = isb.index_score(q8, "e4m3", w.idx_pool, cfg.idx_dtype, w.idx_scale, w.block_table, w.seq_lens,
                             cfg.query_len, cfg.num_kv_heads, cfg.max_blocks)
    torch.cuda.synchronize()
    codes = writer.quantize_query_e4m3(_host(q_bf16))
    assert np.array_equal(q8.cpu().numpy(), codes)
    ref = od.index_score(formats.decode_e4m3(codes), hi["idx_pool"], cfg.idx_dtype, hi["idx_scale"],
                         hi["block_table"], hi["seq_lens"], cfg.query_len, cfg.num_kv_heads, cfg.max_blocks)
    assert_scores_close(scores.cpu().numpy(), ref)


# ------------------------------------------------------------------ a whole decode step
@pytest.mark.parametrize("name", ["fp8_decode", "spec_decode", "mxfp4", "tiny_bf16"])
def test_decode_step_after_the_cache_write(name):
    # A decode step as a server runs it: the step's new tokens written by
    # isb_write_cache (they are each request's last tokens, so every row's tail
    # block holds them), then the layer (index score, select + attend) over the
    # updated caches.  The oracle writes with its own writer into the same
    # starting caches and runs its own layer.
    from _util import check_chain, host_inputs, oracle_layer, small_configs

    cfg = small_configs()[name]
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    T, H, q = cfg.num_tokens, cfg.num_kv_heads, cfg.query_len

    def bf16(*shape):
        return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)

    k_new, v_new, i_new = bf16(T, H, 128), bf16(T, H, 128), bf16(T, 128)
    _say(f"decode step after the write: {name}")
    isb.write_cache(k_new.cuda(), v_new.cuda(), i_new.cuda(), w.block_table, w.seq_lens, q, w.k_pool, w.v_pool,
                    cfg.kv_dtype, w.k_scale, w.v_scale, w.idx_pool, cfg.idx_dtype, w.idx_scale)
    layer = isb.DecodeLayer(w)
    layer.run()
    torch.cuda.synchronize()
    writer.write_cache(_host(k_new), _host(v_new), _host(i_new), hi["block_table"], hi["seq_lens"], q,
                       hi["k_pool"], hi["v_pool"], cfg.kv_dtype, hi["k_scale"], hi["v_scale"], hi["idx_pool"],
                       cfg.idx_dtype, hi["idx_scale"])
    assert np.array_equal(w.k_pool.cpu().numpy(), hi["k_pool"]) and np.array_equal(w.idx_pool.cpu().numpy(),
                                                                                      hi["idx_pool"])
    ref = oracle_layer(hi)
    check_chain(hi, layer.scores.cpu().numpy().astype(np.float64), layer.topk.cpu().numpy(),
                layer.sparse_bt.cpu().numpy(), layer.sparse_ctx.cpu().numpy(), layer.out.float().cpu().numpy(),
                ref, hi["block_table"])


# ------------------------------------------------------------------ QK-norm and rope
def _rope_tables(positions, rot_dim, base=10000.0):
    inv = base ** (-np.arange(0, rot_dim, 2) / rot_dim)
    ang = np.arange(positions)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _exact(x, p, tf):
    """The transform in fp64, not rounded to fp32: the value both sides round."""
    y = np.asarray(x, dtype=np.float64)
    if tf.get("norm_weight") is not None:
        y = writer.rms_norm(y, tf["norm_weight"], tf["eps"])
    if tf.get("cos") is not None:
        y = writer.rope(y, p, tf["cos"], tf["sin"], tf["rot_dim"], tf["neox"])
    return y


def _near_ties_only(got, ref, exact, what):
    """got and ref decoded values agree, except where the exact value sits at a
    tie between them (fp32 arithmetic in a different order may break it either
    way): at most 0.1% of the elements."""
    bad = got != ref
    if bad.any():
        mid = (got[bad] + ref[bad]) / 2
        slack = 2.0 ** -16 * np.maximum(np.abs(exact[bad]), 1e-30)
        assert np.all(np.abs(exact[bad] - mid) <= slack), f"{what}: a mismatch that is not a near tie"
        assert bad.mean() <= 1e-3, f"{what}: {bad.sum()} near ties of {bad.size}"


def _slot_mask(shape, dtype, page_kind, H_kv, slots):
    """Bytes of the written (page, head, slot) triples of a pool, as a mask."""
    m = np.zeros(int(np.prod(shape)), dtype=bool)
    for page, g, slot in slots:
        if dtype == "mxfp4":
            base = (page * (H_kv if page_kind == "kv" else 1) + g) * formats.MXFP4_PAGE_BYTES
            m[base + 64 * slot: base + 64 * slot + 64] = True
            m[base + formats.MXFP4_DATA_BYTES + 4 * slot: base + formats.MXFP4_DATA_BYTES + 4 * slot + 4] = True
        else:
            e = 2 if dtype == "bf16" else 1
            if page_kind == "kv":
                base, c = ((8 * page + slot // 16) * H_kv + g) * 2048 * e, slot % 16
            else:
                base, c = page * 16384 * e + 2048 * e * (slot // 16), slot % 16
            m[base + writer._k_offsets_row(e, c)] = True
    return m.reshape(shape)


NR_CASES = {
    # kv dtype, index dtype, H_kv, query_len, neox, rotated dims, norm on the index key
    "fp8_neox_full": ("fp8", "fp8", 1, 1, True, 128, True),
    "fp8_h2_interleaved_64": ("fp8", "mxfp4", 2, 4, False, 64, False),
    "bf16_neox_32": ("bf16", "bf16", 2, 3, True, 32, True),
    "mxfp4_neox_64": ("mxfp4", "mxfp4", 1, 4, True, 64, True),
}


@pytest.mark.parametrize("name", list(NR_CASES))
def test_write_cache_with_norm_and_rope(name):
    kv, idt, H, q, neox, rot, idx_norm = NR_CASES[name]
    lens = np.array([300, 2, 0, 4097, 129][: 5 if q > 1 else 4], np.int32)
    R = len(lens)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    nblk = 64
    need = [-(-int(L) // 128) for L in lens]
    ids = rng.permutation(nblk)
    bt = rng.integers(0, nblk, (R, 40)).astype(np.int32)
    for r in range(R):
        bt[r, :need[r]] = ids[sum(need[:r]):sum(need[:r + 1])]
    npages = nblk * (8 if kv != "mxfp4" else 1)
    pools = dict(k=rng.integers(0, 256, (npages, H * KV_PAGE[kv]), dtype=np.uint8),
                 v=rng.integers(0, 256, (npages, H * KV_PAGE[kv]), dtype=np.uint8),
                 i=rng.integers(0, 256, (nblk, IDX_PAGE[idt]), dtype=np.uint8))
    T = R * q
    bf = lambda *s: torch.from_numpy((rng.standard_normal(s) * 3).astype(np.float32)).to(torch.bfloat16)  # noqa
    k_new, v_new, i_new = bf(T, H, 128), bf(T, H, 128), bf(T, 128)
    cos, sin = _rope_tables(4200, rot)
    kw = (rng.standard_normal(128) * 0.5 + 1).astype(np.float32)
    iw = (rng.standard_normal(128) * 0.5 + 1).astype(np.float32)
    k_tf = dict(norm_weight=kw, eps=1e-6, cos=cos, sin=sin, rot_dim=rot, neox=neox)
    i_tf = dict(norm_weight=iw if idx_norm else None, eps=1e-6, cos=cos, sin=sin, rot_dim=rot, neox=neox)
    ks, vs, xs = 0.05, 0.021, 0.04
    _say(f"write_cache norm+rope {name}")
    d = {n: torch.from_numpy(a).cuda() for n, a in pools.items()}
    dev_t = {n: torch.from_numpy(a).cuda() for n, a in (("kw", kw), ("iw", iw), ("cos", cos), ("sin", sin))}
    knr = isb.norm_rope(dev_t["kw"], 1e-6, dev_t["cos"], dev_t["sin"], rot, neox)
    inr = isb.norm_rope(dev_t["iw"] if idx_norm else None, 1e-6, dev_t["cos"], dev_t["sin"], rot, neox)
    isb.write_cache(k_new.cuda(), v_new.cuda(), i_new.cuda(), torch.from_numpy(bt).cuda(),
                    torch.from_numpy(lens).cuda(), q, d["k"], d["v"], kv, ks, vs, d["i"], idt, xs,
                    k_norm_rope=knr, idx_norm_rope=inr)
    torch.cuda.synchronize()
    got = {n: t.cpu().numpy() for n, t in d.items()}
    ref = {n: a.copy() for n, a in pools.items()}
    writer.write_cache(_host(k_new), _host(v_new), _host(i_new), bt, lens, q, ref["k"], ref["v"], kv, ks, vs,
                       ref["i"], idt, xs, k_tf=k_tf, idx_tf=i_tf)
    assert np.array_equal(got["v"], ref["v"])                        # V is stored as given
    kslots, islots, toks = [], [], []
    for t in range(T):
        r, i = divmod(t, q)
        p = int(lens[r]) - q + i
        if p < 0:
            continue
        blk = int(bt[r, p // 128])
        toks.append((t, p, blk))
        islots.append((blk, 0, p % 128))
        kslots += [(blk, g, p % 128) for g in range(H)]
    for n, dt, kind, slots in (("k", kv, "kv", kslots), ("i", idt, "idx", islots)):
        outside = ~_slot_mask(got[n].shape, dt, kind, H, slots)
        assert np.array_equal(got[n][outside], ref[n][outside]), f"pool {n} changed outside the written slots"
    for t, p, blk in toks:
        kg = pools_read(got, kv, idt, H, blk, p, ks, xs)
        kr = pools_read(ref, kv, idt, H, blk, p, ks, xs)
        for g in range(H):
            _near_ties_only(kg[0][g], kr[0][g], _exact(_host(k_new)[t, g], p, k_tf), f"K t{t} g{g}")
        _near_ties_only(kg[1], kr[1], _exact(_host(i_new)[t], p, i_tf), f"index key t{t}")


def pools_read(pl, kv, idt, H, blk, p, ks, xs):
    """Decoded K of every head and the index key of position p in block blk."""
    from oracle import pools as op
    if kv == "mxfp4":
        ks_ = [op.kv_page_tokens(pl["k"], pl["v"], kv, [blk], ks, 1.0, head=g, num_kv_heads=H)[0][0, p % 128]
               for g in range(H)]
    else:
        page = 8 * blk + (p % 128) // 16
        ks_ = [op.kv_page_tokens(pl["k"], pl["v"], kv, [page], ks, 1.0, head=g, num_kv_heads=H)[0][0, p % 16]
               for g in range(H)]
    key = op.index_block_keys(pl["i"], idt, xs, [blk])[0][p % 128]
    return ks_, key


@pytest.mark.parametrize("out_dtype", ["e4m3", "bf16"])
@pytest.mark.parametrize("neox,rot", [(True, 128), (False, 64)])
def test_prepare_query_matches_the_oracle(out_dtype, neox, rot):
    rng = np.random.default_rng(rot + neox)
    lens = np.array([70, 1, 0, 40], np.int32)                  # positions 68..69, -1..0, pads, 38..39
    q_len, H = 2, 16
    T = len(lens) * q_len
    qb = torch.from_numpy((rng.standard_normal((T, H, 128)) * 2).astype(np.float32)).to(torch.bfloat16)
    cos, sin = _rope_tables(69, rot)                           # position 69 lies past the table
    w = (rng.standard_normal(128) * 0.3 + 1).astype(np.float32)
    tf = dict(norm_weight=w, eps=1e-5, cos=cos, sin=sin, rot_dim=rot, neox=neox)
    dev = {n: torch.from_numpy(a).cuda() for n, a in (("w", w), ("cos", cos), ("sin", sin))}
    nr = isb.norm_rope(dev["w"], 1e-5, dev["cos"], dev["sin"], rot, neox)
    _say(f"prepare_query {out_dtype} neox {neox} rot {rot}")
    out = isb.prepare_query(qb.cuda(), torch.from_numpy(lens).cuda(), q_len, nr, out_dtype)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16) if out_dtype == "bf16" else out.cpu().numpy()
    dec = (lambda c: torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).double().numpy()) \
        if out_dtype == "bf16" else formats.decode_e4m3
    qh = _host(qb)
    for t in range(T):
        r, i = divmod(t, q_len)
        p = int(lens[r]) - q_len + i
        if p < 0:
            assert not got[t].any()
            continue
        if p >= 69:
            assert np.isnan(dec(got[t])).all()
            continue
        ref = writer.prepare_query(qh[t:t + 1], np.array([p + 1]), 1, tf, "bf16" if out_dtype == "bf16" else "e4m3")
        for h in range(H):
            _near_ties_only(dec(got[t, h]), dec(ref[0, h]), _exact(qh[t, h], p, tf), f"q t{t} h{h}")


@pytest.mark.parametrize("name", ["fp8_decode", "mxfp4"])
def test_fused_decode_step_with_norm_and_rope(name):
    # The whole step with the fused writer's transform: new K and index keys
    # written after QK-norm and rope, the query and the index query prepared
    # with the same (bf16 or e4m3, as the workload's queries are stored), then
    # the layer.  The oracle runs its own writer, query step and layer from the
    # same inputs.  These seeds hit no fp32 near-tie (both sides' codes are
    # equal, checked first), so the chain compares as for any layer.
    from dataclasses import replace as dc_replace

    from _util import check_chain, host_inputs, oracle_layer, small_configs

    cfg = small_configs()[name]
    w = wl.make_workload(cfg, device="cuda")
    hi = host_inputs(w)
    rng = np.random.default_rng(zlib.crc32(name.encode()) + 1)
    T, H, q = cfg.num_tokens, cfg.num_kv_heads, cfg.query_len

    def bf16(*shape):
        return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)

    k_new, v_new, i_new = bf16(T, H, 128), bf16(T, H, 128), bf16(T, 128)
    q_raw, qi_raw = bf16(T, cfg.num_q_heads, 128), bf16(T, cfg.num_idx_heads, 128)
    npos = int(hi["seq_lens"].max())
    cos, sin = _rope_tables(npos, 64)
    wk, wi, wq, wqi = ((rng.standard_normal(128) * 0.2 + 1).astype(np.float32) for _ in range(4))
    tfs = {n: dict(norm_weight=wt, eps=1e-6, cos=cos, sin=sin, rot_dim=64, neox=True)
           for n, wt in (("k", wk), ("i", wi), ("q", wq), ("qi", wqi))}
    dev = {n: torch.from_numpy(a).cuda() for n, a in (("wk", wk), ("wi", wi), ("wq", wq), ("wqi", wqi),
                                                      ("cos", cos), ("sin", sin))}
    nr = {n: isb.norm_rope(dev[wn], 1e-6, dev["cos"], dev["sin"], 64, True)
          for n, wn in (("k", "wk"), ("i", "wi"), ("q", "wq"), ("qi", "wqi"))}
    _say(f"fused decode step with norm + rope: {name}")
    isb.write_cache(k_new.cuda(), v_new.cuda(), i_new.cuda(), w.block_table, w.seq_lens, q, w.k_pool, w.v_pool,
                    cfg.kv_dtype, w.k_scale, w.v_scale, w.idx_pool, cfg.idx_dtype, w.idx_scale,
                    k_norm_rope=nr["k"], idx_norm_rope=nr["i"])
    qg = isb.prepare_query(q_raw.cuda(), w.seq_lens, q, nr["q"], cfg.q_dtype)
    qig = isb.prepare_query(qi_raw.cuda(), w.seq_lens, q, nr["qi"], cfg.qidx_dtype)
    w = dc_replace(w, q=qg.view(torch.uint8), q_idx=qig.view(torch.uint8))
    layer = isb.DecodeLayer(w)
    layer.run()
    torch.cuda.synchronize()
    # the oracle's side
    writer.write_cache(_host(k_new), _host(v_new), _host(i_new), hi["block_table"], hi["seq_lens"], q,
                       hi["k_pool"], hi["v_pool"], cfg.kv_dtype, hi["k_scale"], hi["v_scale"], hi["idx_pool"],
                       cfg.idx_dtype, hi["idx_scale"], k_tf=tfs["k"], idx_tf=tfs["i"])
    q_ref = writer.prepare_query(_host(q_raw), hi["seq_lens"], q, tfs["q"], cfg.q_dtype)
    qi_ref = writer.prepare_query(_host(qi_raw), hi["seq_lens"], q, tfs["qi"], cfg.qidx_dtype)
    assert np.array_equal(w.k_pool.cpu().numpy(), hi["k_pool"]) and np.array_equal(w.idx_pool.cpu().numpy(),
                                                                                      hi["idx_pool"])
    assert np.array_equal(w.q.cpu().numpy(), q_ref.view(np.uint8)) and \
        np.array_equal(w.q_idx.cpu().numpy(), qi_ref.view(np.uint8))
    hi = dict(hi, q=formats.decode_query(q_ref.view(np.uint8), cfg.q_dtype),
              q_idx=formats.decode_query(qi_ref.view(np.uint8), cfg.qidx_dtype))
    ref = oracle_layer(hi)
    check_chain(hi, layer.scores.cpu().numpy().astype(np.float64), layer.topk.cpu().numpy(),
                layer.sparse_bt.cpu().numpy(), layer.sparse_ctx.cpu().numpy(), layer.out.float().cpu().numpy(),
                ref, hi["block_table"])


@pytest.mark.parametrize("name", ["fp8_decode", "mxfp4"])
def test_write_and_layer_replay_from_a_hip_graph(name):
    # A serving loop captures the whole step: the cache write (with QK-norm and
    # rope), the query preparation and the layer.  Between replays the pools go
    # back to their state before the write and every output is overwritten;
    # each replay must give the eager step's pools and outputs bit for bit.
    from dataclasses import replace as dc_replace

    from _util import small_configs

    cfg = small_configs()[name]
    w = wl.make_workload(cfg, device="cuda")
    rng = np.random.default_rng(zlib.crc32(name.encode()) + 2)
    T, H, q = cfg.num_tokens, cfg.num_kv_heads, cfg.query_len

    def bf16(*shape):
        return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16).cuda()

    k_new, v_new, i_new = bf16(T, H, 128), bf16(T, H, 128), bf16(T, 128)
    q_raw = bf16(T, cfg.num_q_heads, 128)
    cos, sin = (torch.from_numpy(a).cuda() for a in _rope_tables(int(w.seq_lens.max().item()), 64))
    wn = torch.from_numpy((rng.standard_normal(128) * 0.2 + 1).astype(np.float32)).cuda()
    nr = isb.norm_rope(wn, 1e-6, cos, sin, 64, True)
    q_out = torch.empty((T, cfg.num_q_heads, 128), dtype=torch.bfloat16 if cfg.q_dtype == "bf16" else torch.uint8,
                        device="cuda")
    w = dc_replace(w, q=q_out.view(torch.uint8))
    layer = isb.DecodeLayer(w)
    pools0 = [t.clone() for t in (w.k_pool, w.v_pool, w.idx_pool)]

    def step():
        isb.write_cache(k_new, v_new, i_new, w.block_table, w.seq_lens, q, w.k_pool, w.v_pool, cfg.kv_dtype,
                        w.k_scale, w.v_scale, w.idx_pool, cfg.idx_dtype, w.idx_scale, k_norm_rope=nr,
                        idx_norm_rope=nr)
        isb.prepare_query(q_raw, w.seq_lens, q, nr, cfg.q_dtype, out=q_out)
        layer.run()

    _say(f"graph of write + layer: {name}")
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (w.k_pool, w.v_pool, w.idx_pool, q_out, layer.topk, layer.out)]
    for t, t0 in zip((w.k_pool, w.v_pool, w.idx_pool), pools0):
        t.copy_(t0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capturing stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t, t0 in zip((w.k_pool, w.v_pool, w.idx_pool), pools0):
            t.copy_(t0)                    # eager work between replays
        q_out.zero_()
        layer.out.fill_(float("nan"))
        layer.topk.fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (w.k_pool, w.v_pool, w.idx_pool, q_out, layer.topk, layer.out)
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               b.view(torch.uint8) if b.dtype != torch.int32 else b), f"replay {rep}"
    del graph
    torch.cuda.synchronize()
