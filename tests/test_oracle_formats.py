"""Pins for the oracle's element and page decoders (CPU only).

Each decoder is checked against something other than itself: torch's own dtype
conversions (a library routine) over every code, the closed-form OCP MX value
table, and sizes the source pages print (tests/golden/page_arithmetic.json).
"""
import json
import math
import os

import numpy as np
import torch

from oracle import formats, pools

import _pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_e4m3_every_code_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.decode_e4m3(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2                                # 0x7F and 0xFF
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9   # max normal, min subnormal


def test_e8m0_every_code_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = formats.decode_e8m0(np.arange(256, dtype=np.uint8))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])
    assert got[127] == 1.0 and got[123] == 1 / 16 and got[131] == 16.0


def test_e2m1_closed_form_table():
    # OCP MX v1.0 FP4 (E2M1) values for codes 0..7; codes 8..15 are the negatives.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = formats.decode_e2m1(np.arange(16, dtype=np.uint8))
    assert list(got[:8]) == mags
    assert list(-got[8:]) == mags
    assert np.signbit(got[8])                            # -0


def test_e2m1_against_e4m3_bit_remap():
    # Independent route: an e2m1 code (s, E, m) with E >= 1 has the value of the
    # e4m3 code with exponent E + 6 and mantissa m << 2; e2m1 0.5 is e4m3 0x30.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:
            e4 = 0x30 if m else 0x00
        else:
            e4 = ((e + 6) << 3) | (m << 2)
        e4 |= s << 7
        ref = torch.tensor([e4], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        assert formats.decode_e2m1(np.array([c]))[0] == ref


def test_bf16_every_code_matches_torch():
    u16 = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = u16.view(torch.bfloat16).to(torch.float64).numpy()
    got = formats.decode_bf16_bytes(u16.numpy().view(np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_mxfp4_page_size_is_the_printed_one():
    g = _golden()
    page = g["mxfp4_page_bytes"]
    assert formats.MXFP4_PAGE_BYTES == page["value"]
    assert page["data"][0] * page["data"][1] + page["scales"][0] * page["scales"][1] == page["value"]
    # one e8m0 per 32 e2m1 elements of 128 dims: 64 B + 4 B a token
    assert formats.MXFP4_PAGE_BYTES // 128 == g["bytes_per_token"]["index"]
    assert 2 * formats.MXFP4_PAGE_BYTES // 128 == g["bytes_per_token"]["kv"]
    # the fp4 pool's per-block bytes are a whole number of pages, and the
    # allocation the page reports is that count times the block bytes
    blk = g["pool_block_bytes_fp4"]
    assert blk["block_bytes"] % formats.MXFP4_PAGE_BYTES == 0
    assert math.isclose(blk["blocks"] * blk["block_bytes"] / 2**30, blk["gib"], abs_tol=5e-4)


def test_fp8_page16_bytes_match_the_printed_shapes():
    # Our fp8 K and V pages (16 tokens x 128 dims, 2048 B each, in our own
    # element order) hold as many bytes as one entry of the printed
    # K [.., 8, 16, 16] and V [.., 1, 128, 16], and the pool file holds them.
    g = _golden()["fp8_page16_shapes"]
    assert math.prod(g["k_cache"][1:]) == 16 * 128
    assert math.prod(g["v_cache"][1:]) == 128 * 16
    from indexer_selected_block_amd import workload as wl
    assert wl.kv_page_bytes("fp8") == math.prod(g["k_cache"][1:])


def test_mxfp4_page_hand_built():
    page = np.zeros(formats.MXFP4_PAGE_BYTES, dtype=np.uint8)
    page[8192:] = 127                                   # all scales 2^0
    # token 5: dim 6 = +1.5 (code 3, low nibble of byte 3), dim 7 = -6 (code 15, high nibble)
    page[64 * 5 + 3] = 0x3 | (0xF << 4)
    page[8192 + 4 * 5 + 0] = 127 + 2                    # dims 0..31 of token 5 scaled by 4
    # token 127, dim 127 = 0.5 (code 1, high nibble of byte 63) with scale 2^-3 (dims 96..127)
    page[64 * 127 + 63] = 0x1 << 4
    page[8192 + 4 * 127 + 3] = 127 - 3
    v = formats.decode_mxfp4_page(page)
    assert v.shape == (128, 128)
    assert v[5, 6] == 6.0 and v[5, 7] == -24.0
    assert v[127, 127] == 0.5 / 8
    nz = np.argwhere(v != 0)
    assert sorted(map(tuple, nz)) == [(5, 6), (5, 7), (127, 127)]
    page[8192 + 4 * 9 + 1] = 0xFF                       # NaN scale poisons dims 32..63 of token 9
    v = formats.decode_mxfp4_page(page)
    assert np.isnan(v[9, 32:64]).all() and not np.isnan(v[9, :32]).any()


def test_pool_readers_match_torch_views():
    # The pool readers against torch's own reinterpretation of the same bytes,
    # laid out lane by lane (tests/_pages.py): index blocks as eight K-page
    # tiles, K and V pages, for fp8 and bf16.
    rng = np.random.default_rng(0)
    vals = torch.from_numpy(rng.standard_normal((3, 128, 128)).astype(np.float32))
    tiles = lambda t: _pages.k_pages(t.view(torch.uint8).numpy().reshape(24, 16, 128, t.element_size())).reshape(3, -1)  # noqa: E731
    idx_bf16 = tiles(vals.to(torch.bfloat16))
    got = pools.index_block_keys(idx_bf16, "bf16", 1.0, [2, 0])
    assert np.array_equal(got, vals.to(torch.bfloat16).double().numpy()[[2, 0]])
    idx_fp8 = (vals / 4).to(torch.float8_e4m3fn)
    got = pools.index_block_keys(tiles(idx_fp8), "fp8", 0.5, [1])
    assert np.array_equal(got[0], idx_fp8.double().numpy()[1] * 0.5)
    k = (vals[:, :16] / 4).to(torch.float8_e4m3fn)            # [3 pages, 16 tok, 128 dim]
    v = (vals[:, 16:32] / 4).to(torch.float8_e4m3fn)
    k_pool = _pages.k_pages(k.view(torch.uint8).numpy().reshape(3, 16, 128, 1))
    v_pool = _pages.v_pages(v.view(torch.uint8).numpy().reshape(3, 16, 128, 1))
    K, V = pools.kv_page_tokens(k_pool, v_pool, "fp8", [2, 1], 2.0, 3.0)
    assert np.array_equal(K, k.double().numpy()[[2, 1]] * 2.0)
    assert np.array_equal(V, v.double().numpy()[[2, 1]] * 3.0)
    kb = vals[:, 32:48].to(torch.bfloat16)
    vb = vals[:, 48:64].to(torch.bfloat16)
    k_pool = _pages.k_pages(kb.view(torch.uint8).numpy().reshape(3, 16, 128, 2))
    v_pool = _pages.v_pages(vb.view(torch.uint8).numpy().reshape(3, 16, 128, 2))
    K, V = pools.kv_page_tokens(k_pool, v_pool, "bf16", [0, 2], 1.0, 1.0)
    assert np.array_equal(K, kb.double().numpy()[[0, 2]])
    assert np.array_equal(V, vb.double().numpy()[[0, 2]])
    # two KV heads under one page id: row g reads head g's page
    k2 = np.concatenate([_pages.k_pages(k.view(torch.uint8).numpy().reshape(3, 16, 128, 1)),
                         _pages.k_pages(v.view(torch.uint8).numpy().reshape(3, 16, 128, 1))], axis=1)
    K0, _ = pools.kv_page_tokens(k2, k2, "fp8", [1], 1.0, 1.0, head=0, num_kv_heads=2)
    K1, _ = pools.kv_page_tokens(k2, k2, "fp8", [1], 1.0, 1.0, head=1, num_kv_heads=2)
    assert np.array_equal(K0[0], k.double().numpy()[1]) and np.array_equal(K1[0], v.double().numpy()[1])


def test_generator_page_layout_matches_lane_builder():
    # The generator's tensor permutes and the lane-by-lane builder agree.
    from indexer_selected_block_amd import workload as wl
    rng = np.random.default_rng(3)
    for e in (1, 2):
        vals = rng.integers(0, 256, (5, 16, 128, e), dtype=np.uint8)
        t = torch.from_numpy(vals)
        assert np.array_equal(wl.k_page16_bytes(t).numpy(), _pages.k_pages(vals))
        assert np.array_equal(wl.v_page16_bytes(t).numpy(), _pages.v_pages(vals))
        assert np.array_equal(_pages.read_back(_pages.k_pages(vals), e, "k"), vals)
        assert np.array_equal(_pages.read_back(_pages.v_pages(vals), e, "v"), vals)
