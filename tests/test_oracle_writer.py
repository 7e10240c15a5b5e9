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


def _double_rounding_cases():
    """(x, scale) pairs, x a bf16 value and scale an fp32 number, whose fp32
    quotient fl32(x / scale) lands exactly on the midpoint between two
    adjacent e4m3 values while the exact quotient lies off it, so that rounding
    the exact quotient and rounding the fp32 quotient give different codes.
    Built from the midpoints of torch's own e4m3 value table, independent of
    the oracle's tables."""
    from fractions import Fraction
    vals = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    out = []
    for c in range(8, 0x7E):
        mid = Fraction(vals[c]) / 2 + Fraction(vals[c + 1]) / 2
        for x in (0.1171875, 0.75, 1.0, 1.5, 3.25, 7.0, 13.5, 100.0):
            base = np.float32(float(Fraction(x) / mid))
            for step in range(-3, 4):
                s = np.nextafter(base, np.float32(np.inf if step > 0 else 0), dtype=np.float32)
                for _ in range(abs(step) - 1):
                    s = np.nextafter(s, np.float32(np.inf if step > 0 else 0), dtype=np.float32)
                s = base if step == 0 else s
                q32 = np.float32(np.float32(x) / s)
                exact = Fraction(x) / Fraction(float(s))
                if Fraction(float(q32)) != mid or exact == mid:
                    continue
                out.append((x, float(s), c, exact > mid))
    return out


def test_scaled_e4m3_is_the_rounding_of_the_fp32_quotient():
    # The library's quantiser with a per-tensor scale: the code of fl32(x / scale),
    # rounded to nearest with ties to even.  Where that differs from rounding the
    # exact quotient (double-rounding cases), the oracle must follow the stated
    # definition, and so must torch's own fp32 division followed by its e4m3 cast.
    cases = _double_rounding_cases()
    differ = 0
    for x, s, c, above in cases:
        got = int(writer.quantize_e4m3_scaled(np.float64(x), s))
        ties_even = c if c % 2 == 0 else c + 1                 # the tie at the midpoint: even code
        exact = c + 1 if above else c                           # nearest to the exact quotient
        lib = int((torch.tensor([x], dtype=torch.float32) / torch.tensor([s], dtype=torch.float32))
                  .to(torch.float8_e4m3fn).view(torch.uint8)[0])
        assert got == ties_even == lib, (x, s, c)
        differ += exact != got
    assert differ >= 100, f"only {differ} cases separate the two roundings"
    # and the cache writer stores exactly these codes (one fp8 key per case)
    for x, s, c, _ in cases[:64]:
        k_pool = np.zeros((8, 2048), dtype=np.uint8)
        v_pool = np.zeros((8, 2048), dtype=np.uint8)
        idx_pool = np.zeros((1, 16384), dtype=np.uint8)
        k = np.full((1, 1, 128), x)
        writer.write_cache(k, k, None, np.array([[0]]), np.array([1]), 1, k_pool, v_pool, "fp8", s, s,
                           idx_pool, "fp8", 1.0)
        K, _ = pools.kv_page_tokens(k_pool, v_pool, "fp8", [0], 1.0, 1.0)
        code = int(writer.encode_e4m3(K[0, 0, 0]))
        assert code == (c if c % 2 == 0 else c + 1)


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


# ------------------------------------------------------------------ QK-norm and rope
def _tables(positions, rot_dim, base=10000.0):
    inv = base ** (-np.arange(0, rot_dim, 2) / rot_dim)
    ang = np.arange(positions)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32), ang


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 128)) * 3
    w = rng.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.allclose(writer.rms_norm(x, w, 1e-6), ref, rtol=1e-13, atol=1e-13)
    # unit weight, no epsilon: unit root mean square, and a scaled input gives the same output
    y = writer.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    assert np.allclose(writer.rms_norm(5 * x, np.ones(128), 0.0), y, rtol=1e-13)


@pytest.mark.parametrize("rot_dim", [128, 64, 32])
def test_rope_neox_is_a_complex_rotation_and_interleaved_its_permutation(rot_dim):
    rng = np.random.default_rng(rot_dim)
    cos, sin, _ = _tables(40, rot_dim)
    half = rot_dim // 2
    for pos in (0, 1, 17, 39):
        x = rng.standard_normal(128)
        z = (x[:half] + 1j * x[half:rot_dim]) * (cos[pos].astype(np.float64) + 1j * sin[pos].astype(np.float64))
        y = writer.rope(x, pos, cos, sin, rot_dim, neox=True)
        assert np.allclose(y[:half], z.real, rtol=0, atol=1e-14) and np.allclose(y[half:rot_dim], z.imag, atol=1e-14)
        assert np.array_equal(y[rot_dim:], x[rot_dim:])
        # interleaved pairs (2i, 2i+1) are NeoX pairs after moving even dims first
        perm = np.concatenate([np.arange(0, rot_dim, 2), np.arange(1, rot_dim, 2), np.arange(rot_dim, 128)])
        yi = writer.rope(x, pos, cos, sin, rot_dim, neox=False)
        assert np.allclose(yi[perm], writer.rope(x[perm], pos, cos, sin, rot_dim, neox=True), atol=1e-14)
    # position 0 turns nothing; turning by p then by q is turning by p + q
    x = rng.standard_normal(128)
    assert np.allclose(writer.rope(x, 0, cos, sin, rot_dim, True), x, atol=1e-15)
    c64, s64 = np.cos(_tables(40, rot_dim)[2]), np.sin(_tables(40, rot_dim)[2])
    two = writer.rope(writer.rope(x, 5, c64, s64, rot_dim, True), 7, c64, s64, rot_dim, True)
    assert np.allclose(two, writer.rope(x, 12, c64, s64, rot_dim, True), atol=1e-12)


def test_bf16_bits_round_to_nearest_even_like_torch():
    rng = np.random.default_rng(6)
    b = torch.from_numpy(rng.standard_normal(4000).astype(np.float32)).to(torch.bfloat16).float().numpy()
    step = np.abs(b) * 2.0 ** -8                          # half a bf16 step at each value
    x = np.concatenate([rng.standard_normal(20000) * 50, b + step, b - step, [np.inf, -np.inf, 0.0, -0.0]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(writer.bf16_bits(x), ref)


@pytest.mark.parametrize("kv_dtype,idx_dtype,neox", [("fp8", "mxfp4", True), ("bf16", "fp8", False),
                                                     ("mxfp4", "bf16", True)])
def test_writer_with_norm_and_rope_stores_the_transformed_keys(kv_dtype, idx_dtype, neox):
    rng = np.random.default_rng(7)
    H_kv, q_len = 2, 2
    seq_lens = np.array([300, 1])
    bt = np.array([[2, 0, 3], [1, 3, 3]])
    nblk = 4
    kpb = {"bf16": 4096, "fp8": 2048}.get(kv_dtype, formats.MXFP4_PAGE_BYTES)
    ipb = {"bf16": 32768, "fp8": 16384, "mxfp4": formats.MXFP4_PAGE_BYTES}[idx_dtype]
    npages = nblk * (8 if kv_dtype != "mxfp4" else 1)
    k_pool = np.zeros((npages, H_kv * kpb), np.uint8)
    v_pool = np.zeros_like(k_pool)
    idx_pool = np.zeros((nblk, ipb), np.uint8)
    T = 2 * q_len
    k_new, v_new, idx_new = rng.standard_normal((T, H_kv, 128)), rng.standard_normal((T, H_kv, 128)), \
        rng.standard_normal((T, 128))
    cos, sin, _ = _tables(512, 64)
    k_tf = dict(norm_weight=rng.standard_normal(128), eps=1e-6, cos=cos, sin=sin, rot_dim=64, neox=neox)
    i_tf = dict(norm_weight=None, eps=0.0, cos=cos, sin=sin, rot_dim=64, neox=neox)
    ks, vs, xs = 0.02, 0.03, 0.05
    writer.write_cache(k_new, v_new, idx_new, bt, seq_lens, q_len, k_pool, v_pool, kv_dtype, ks, vs,
                       idx_pool, idx_dtype, xs, k_tf=k_tf, idx_tf=i_tf)
    plain_k, plain_v, plain_i = k_pool.copy(), v_pool.copy(), idx_pool.copy()
    # the same pools written without the transform from the transformed vectors
    kt = np.array([[writer.transform(k_new[t, g], seq_lens[t // q_len] - q_len + t % q_len, k_tf)
                    for g in range(H_kv)] for t in range(T)])
    it = np.array([writer.transform(idx_new[t], max(0, seq_lens[t // q_len] - q_len + t % q_len), i_tf)
                   for t in range(T)])
    k2, v2, i2 = np.zeros_like(k_pool), np.zeros_like(v_pool), np.zeros_like(idx_pool)
    writer.write_cache(kt, v_new, it, bt, seq_lens, q_len, k2, v2, kv_dtype, ks, vs, i2, idx_dtype, xs)
    assert np.array_equal(plain_k, k2) and np.array_equal(plain_v, v2) and np.array_equal(plain_i, i2)
    # and rope moved the keys: without it the pools differ
    k3, v3, i3 = np.zeros_like(k_pool), np.zeros_like(v_pool), np.zeros_like(idx_pool)
    writer.write_cache(k_new, v_new, idx_new, bt, seq_lens, q_len, k3, v3, kv_dtype, ks, vs, i3, idx_dtype, xs)
    assert not np.array_equal(k3, plain_k) and not np.array_equal(i3, plain_i) and np.array_equal(v3, plain_v)


def test_prepare_query_pads_zero_and_casts_the_transformed_rows():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 3, 128)) * 2
    seq_lens = np.array([50, 1])
    cos, sin, _ = _tables(64, 128)
    tf = dict(norm_weight=np.full(128, 0.5), eps=1e-5, cos=cos, sin=sin, rot_dim=128, neox=True)
    out8 = writer.prepare_query(q, seq_lens, 2, tf, "e4m3")
    out16 = writer.prepare_query(q, seq_lens, 2, tf, "bf16")
    assert not out8[2].any() and not out16[2].any()                 # request 1, token 0: position -1
    for t, p in ((0, 48), (1, 49), (3, 0)):
        y = np.array([writer.transform(q[t, h], p, tf) for h in range(3)])
        assert np.array_equal(out8[t], writer.encode_e4m3(y)) and np.array_equal(out16[t], writer.bf16_bits(y))
    # without a transform the e4m3 output is the plain cast
    assert np.array_equal(writer.prepare_query(q, np.array([2, 2]), 2, None, "e4m3"), writer.quantize_query_e4m3(q))
