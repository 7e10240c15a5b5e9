"""Pins for the oracle's cache writer and e4m3 query cast (CPU only).

The encoders are checked against torch's float8_e4m3fn conversion (a library
routine, round to nearest even) on values that include every midpoint between
adjacent codes, against brute force over the e2m1 values, and by round trips;
the writer is checked against the oracle's own page readers: what it writes
reads back as the encoded values at the token's position, and nothing else in
the pools changes.
"""
import numpy as np
import pytest
import torch

from oracle import formats, pools, writer


def test_e4m3_encode_matches_torch_including_ties():
    vals = np.array([formats.e4m3_value(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2                      # every tie between neighbours
    rng = np.random.default_rng(0)
    x = np.concatenate([vals, mids, rng.uniform(0, 448, 20000), rng.standard_normal(20000) * 3])
    x = np.concatenate([x, -x])
    got = writer.encode_e4m3(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_keeps_sign_and_nan():
    got = writer.encode_e4m3([448.0, 460.0, 1e6, -1e6, np.inf, -np.inf, np.nan, -0.0, -1e-12])
    assert list(got) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0x80, 0x80]


def test_e4m3_round_trip_of_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(writer.encode_e4m3(formats.decode_e4m3(codes)), codes)


def test_e2m1_encode_is_the_nearest_value_ties_to_even():
    mags = [formats.e2m1_value(c) for c in range(8)]
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-7, 7, 5000), [(a + b) / 2 for a, b in zip(mags, mags[1:])], mags])
    got = writer.encode_e2m1(x)
    for xi, ci in zip(x, got):
        a = min(abs(xi), 6.0)
        d = [abs(a - m) for m in mags]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert ci == want | (8 if np.signbit(xi) else 0), xi


def test_mx_quantize_exponent_and_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)) * np.exp2(rng.integers(-8, 8, (50, 1)))
    x[0, :32] = 0.0                                          # an all-zero group
    codes, scales = writer.mx_quantize(x)
    e = scales.astype(np.int64) - 127
    assert e[0, 0] == -127
    g = x.reshape(50, 4, 32)
    amax = np.abs(g).max(axis=-1)
    nz = amax > 0
    # the group maximum lands in [4, 8) of the scale (saturating to 6 above 6)
    assert np.all((amax[nz] / np.exp2(e[nz]) >= 4) & (amax[nz] / np.exp2(e[nz]) < 8))
    dec = formats.decode_e2m1(codes).reshape(50, 4, 32) * np.exp2(e)[..., None]
    # every element within half a step of its e2m1 value, or saturated at 6 scale
    step = np.exp2(e)[..., None]
    a = np.minimum(np.abs(g) / step, 6.0)
    err = np.abs(np.minimum(np.abs(g), 6 * step) - np.abs(dec))
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0)) * step
    assert np.all(err <= half + 1e-300)


@pytest.mark.parametrize("kv_dtype,idx_dtype", [("fp8", "fp8"), ("bf16", "bf16"), ("mxfp4", "mxfp4"),
                                                ("fp8", "mxfp4")])
def test_writer_reads_back_through_the_page_readers(kv_dtype, idx_dtype):
    rng = np.random.default_rng(3)
    H_kv, q_len = 2, 3
    seq_lens = np.array([130, 2, 17])                        # request 1 is shorter than the chunk
    nblk = 6
    bt = np.array([[4, 1, 5], [0, 5, 5], [2, 3, 5]])
    T = 3 * q_len
    kpb = {"bf16": 4096, "fp8": 2048}.get(kv_dtype, formats.MXFP4_PAGE_BYTES)
    ipb = {"bf16": 32768, "fp8": 16384, "mxfp4": formats.MXFP4_PAGE_BYTES}[idx_dtype]
    npages = nblk * (8 if kv_dtype != "mxfp4" else 1)
    k_pool = rng.integers(0, 256, (npages, H_kv * kpb), dtype=np.uint8)
    v_pool = rng.integers(0, 256, (npages, H_kv * kpb), dtype=np.uint8)
    idx_pool = rng.integers(0, 256, (nblk, ipb), dtype=np.uint8)
    k0, v0, i0 = k_pool.copy(), v_pool.copy(), idx_pool.copy()
    vals = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(torch.bfloat16).double().numpy()  # noqa: E731
    k_new, v_new, idx_new = vals(T, H_kv, 128), vals(T, H_kv, 128), vals(T, 128)
    ks, vs, xs = 0.02, 0.03, 0.05
    writer.write_cache(k_new, v_new, idx_new, bt, seq_lens, q_len, k_pool, v_pool, kv_dtype, ks, vs,
                       idx_pool, idx_dtype, xs)

    def stored(x, dtype, scale):
        if dtype == "bf16":
            return x
        if dtype == "fp8":
            y = (x.astype(np.float32) / np.float32(scale)).astype(np.float64)
            return formats.decode_e4m3(writer.encode_e4m3(y)) * scale
        c, sc = writer.mx_quantize(x)
        return formats.decode_e2m1(c) * np.repeat(formats.decode_e8m0(sc), 32, axis=-1)

    touched_k, touched_i = set(), set()
    for t in range(T):
        r, i = divmod(t, q_len)
        p = seq_lens[r] - q_len + i
        if p < 0:
            continue
        blk = bt[r][p // 128]
        keys = pools.index_block_keys(idx_pool, idx_dtype, xs, [blk])[0]
        assert np.array_equal(keys[p % 128], stored(idx_new[t], idx_dtype, xs))
        touched_i.add(blk)
        page = 8 * blk + (p % 128) // 16 if kv_dtype != "mxfp4" else blk
        slot = p % 16 if kv_dtype != "mxfp4" else p % 128
        for g in range(H_kv):
            K, V = pools.kv_page_tokens(k_pool, v_pool, kv_dtype, [page], ks, vs, head=g, num_kv_heads=H_kv)
            assert np.array_equal(K[0, slot], stored(k_new[t, g], kv_dtype, ks))
            assert np.array_equal(V[0, slot], stored(v_new[t, g], kv_dtype, vs))
        touched_k.add(page)
    # pages no token was written to are byte-identical
    for n in range(npages):
        if n not in touched_k:
            assert np.array_equal(k_pool[n], k0[n]) and np.array_equal(v_pool[n], v0[n])
    for n in range(nblk):
        if n not in touched_i:
            assert np.array_equal(idx_pool[n], i0[n])


def test_writer_without_index_key_leaves_the_index_pool_and_writes_the_same_kv():
    rng = np.random.default_rng(4)
    bt, seq_lens = np.array([[1, 0]]), np.array([200])
    k_new, v_new = rng.standard_normal((2, 2, 1, 128))          # two tokens, one KV head each
    idx_new = rng.standard_normal((2, 128))
    pools_a = [np.zeros((16, 2048), np.uint8), np.zeros((16, 2048), np.uint8), np.zeros((2, 16384), np.uint8)]
    pools_b = [a.copy() for a in pools_a]
    writer.write_cache(k_new, v_new, idx_new, bt, seq_lens, 2, pools_a[0], pools_a[1], "fp8", 0.1, 0.1,
                       pools_a[2], "fp8", 0.1)
    writer.write_cache(k_new, v_new, None, bt, seq_lens, 2, pools_b[0], pools_b[1], "fp8", 0.1, 0.1,
                       pools_b[2], "fp8", 0.1)
    assert np.array_equal(pools_a[0], pools_b[0]) and np.array_equal(pools_a[1], pools_b[1])
    assert pools_a[2].any() and not pools_b[2].any()


def test_query_cast_is_unit_scale_saturating_e4m3():
    q = np.array([1.0, -2.5, 500.0, 0.0])
    assert list(writer.quantize_query_e4m3(q)) == [0x38, 0xC2, 0x7E, 0x00]
