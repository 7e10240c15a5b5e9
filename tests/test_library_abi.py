"""The C ABI on the CPU: the library loads, exports every symbol include/isb.h
declares, and rejects bad arguments before touching a GPU.  No kernel runs here."""
import ctypes
import os
import re

import pytest

from indexer_selected_block_amd import binding
from indexer_selected_block_amd.build import LIB_PATH, build_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isb.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        build_library()
    return binding.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(isb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("isb_index_score", "isb_topk_select", "isb_emit_sparse_block_table",
              "isb_sparse_pa_decode", "isb_sparse_pa_workspace_bytes", "isb_strerror", "isb_version",
              "isb_sparse_pa_decode_noalloc",
              "isb_write_cache", "isb_quantize_e4m3", "isb_prepare_query", "isb_topk_merge",
              "isb_index_score_prefill", "isb_topk_select_prefill", "isb_emit_sparse_block_table_prefill",
              "isb_topk_select_emit_prefill", "isb_sparse_pa_prefill", "isb_select_attend_prefill"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(binding.EXPORTED)


def test_measurement_library_exports_its_header(lib):
    # libisb_ceiling: the benchmark's page-read ceilings, declared in
    # include/isb_ceiling.h, built beside libisb; argument checks on the CPU
    from indexer_selected_block_amd.build import CEILING_LIB_PATH, build_ceiling_library
    if not os.path.exists(CEILING_LIB_PATH):
        build_ceiling_library()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "isb_ceiling.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(isb_[a-z0-9_]+)\s*\(", text)))
    assert names == ["isb_ceiling_attention_gather", "isb_ceiling_attention_words", "isb_ceiling_index_gather"]
    ceil = ctypes.CDLL(CEILING_LIB_PATH)
    for n in names:
        assert hasattr(ceil, n)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    ceil.isb_ceiling_index_gather.argtypes = [P, P, I, I64, P, I, P, I, I, I, I, P]
    ceil.isb_ceiling_attention_gather.argtypes = [P, P, P, I, I64, P, I, P, I, I, I, P, ctypes.c_size_t]
    ceil.isb_ceiling_attention_words.argtypes = [I, I, I, I]
    ceil.isb_ceiling_attention_words.restype = ctypes.c_size_t
    assert ceil.isb_ceiling_attention_words(128, 1, 128, 1) == 128 * 2 * 8     # 2 splits of 8 waves
    assert ceil.isb_ceiling_attention_words(0, 1, 128, 1) == 0
    p = ctypes.c_void_p(16)
    assert ceil.isb_ceiling_index_gather(None, None, 1, 8, p, 4, p, 1, 1, 1, 4, p) == -1
    assert ceil.isb_ceiling_index_gather(None, p, 5, 8, p, 4, p, 1, 1, 1, 4, p) == -2
    assert ceil.isb_ceiling_index_gather(None, p, 1, 8, p, 4, p, 1, 17, 1, 4, p) == -3     # prefill chunk
    assert ceil.isb_ceiling_attention_gather(None, p, p, 1, 8, p, 128, p, 3, 2, 1, p, 1 << 20) == -3
    assert ceil.isb_ceiling_attention_gather(None, p, p, 1, 8, p, 128, p, 128, 1, 1, p, 100) == -4


def test_version_and_strerror(lib):
    assert lib.isb_version() >= 100
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.isb_strerror(s)
    assert b"unknown" in lib.isb_strerror(-99)


NULL = None


def test_argument_checks_return_before_any_launch(lib):
    # null pointers
    assert lib.isb_index_score(NULL, NULL, 0, 1, NULL, 0, 1.0, 1, NULL, 1, NULL, 1, 1, 1, 1, NULL) == -1
    assert lib.isb_topk_select(NULL, NULL, NULL, 1, 1, 1, 1, 1, NULL) == -1
    assert lib.isb_emit_sparse_block_table(NULL, NULL, NULL, 1, NULL, 1, 1, 1, 1, 8, NULL, NULL) == -1
    assert lib.isb_topk_select_emit(NULL, NULL, NULL, 1, 1, 1, 4, 2, NULL, 4, 8, NULL, NULL, NULL) == -1
    assert lib.isb_select_attend(NULL, NULL, NULL, 1, 1, 1, 4, 2, NULL, 4, NULL, 0, NULL, NULL, 1, 8, 1.0, 1.0,
                                 16, 0.1, NULL, 0, NULL, NULL, NULL, NULL) == -1
    assert lib.isb_sparse_pa_decode(NULL, NULL, 0, NULL, NULL, 1, 1, 1.0, 1.0, NULL, 1, NULL, 1, 1, 16, 1,
                                    128, 0.1, NULL, 0, NULL) == -1
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails its checks first
    # dtypes
    assert lib.isb_index_score(NULL, p, 7, 1, p, 0, 1.0, 1, p, 1, p, 1, 1, 1, 1, p) == -2
    assert lib.isb_index_score(NULL, p, 2, 1, p, 0, 1.0, 1, p, 1, p, 1, 1, 1, 1, p) == -2   # MXFP4 query
    assert lib.isb_sparse_pa_decode(NULL, p, 0, p, p, 9, 1, 1.0, 1.0, p, 1, p, 1, 1, 16, 1, 128, 0.1,
                                    p, 1 << 20, p) == -2
    # shapes
    assert lib.isb_index_score(NULL, p, 0, 3, p, 0, 1.0, 1, p, 4, p, 1, 1, 2, 4, p) == -3       # 3 % 2
    assert lib.isb_index_score(NULL, p, 0, 1, p, 0, 1.0, 1, p, 4, p, 1, 1, 1, 5, p) == -3       # MB > stride
    assert lib.isb_topk_select(NULL, p, p, 1, 1, 1, 4, 5, p) == -3                              # K > MB
    assert lib.isb_topk_select(NULL, p, p, 1, 1, 1, 4, 0, p) == -3
    assert lib.isb_emit_sparse_block_table(NULL, p, p, 4, p, 1, 1, 1, 4, 4, p, p) == -3          # ppb 4
    assert lib.isb_topk_select_emit(NULL, p, p, 1, 1, 1, 4, 2, p, 4, 4, p, p, p) == -3            # ppb 4
    assert lib.isb_topk_select_emit(NULL, p, p, 1, 1, 1, 8, 2, p, 4, 8, p, p, p) == -3            # MB > stride
    assert lib.isb_topk_select_emit(NULL, p, p, 1, 1, 1, 4, 5, p, 4, 8, p, p, p) == -3            # K > MB
    # more than 16 tokens or 64 query rows take the wide scorer, whose 16-row
    # tiles must hold whole tokens: 16 % H_idx == 0
    assert lib.isb_index_score(NULL, p, 0, 3, p, 0, 1.0, 1, p, 4, p, 1, 17, 1, 4, p) == -3      # q 17, H_idx 3
    assert lib.isb_index_score(NULL, p, 0, 3, p, 0, 1.0, 1, p, 4, p, 1, 22, 3, 4, p) == -3      # 66 rows, H_idx 3
    assert lib.isb_index_score(NULL, p, 0, 16, p, 0, 1.0, 1, p, 4, p, 1, 65537, 1, 4, p) == -3  # rows > 2^20
    assert lib.isb_index_score(NULL, p, 0, 1, p, 0, 1.0, 1, p, 4, p, 65535, 40000, 1, 4, p) == -3  # T > 2^31-1
    assert lib.isb_select_attend(NULL, p, p, 1, 1, 1, 8, 2, p, 4, p, 0, p, p, 1, 8, 1.0, 1.0,
                                 16, 0.1, p, 1 << 20, p, p, p, p) == -3                          # MB > stride
    assert lib.isb_select_attend(NULL, p, p, 1, 1, 1, 4, 2, p, 4, p, 0, p, p, 1, 8, 1.0, 1.0,
                                 32, 0.1, p, 1 << 20, p, p, p, p) == -3                          # G = 32
    assert lib.isb_select_attend(NULL, p, p, 1, 1, 1, 8, 8, p, 8, p, 0, p, p, 1, 8, 1.0, 1.0,
                                 16, 0.1, p, 16, p, p, p, p) == -4                               # workspace
    assert lib.isb_sparse_pa_decode(NULL, p, 0, p, p, 1, 8, 1.0, 1.0, p, 8, p, 1, 1, 16, 1, 64, 0.1,
                                    p, 1 << 20, p) == -3                                         # head_dim
    assert lib.isb_sparse_pa_decode(NULL, p, 0, p, p, 1, 8, 1.0, 1.0, p, 8, p, 1, 1, 32, 1, 128, 0.1,
                                    p, 1 << 20, p) == -3                                         # G = 32
    # the cache writer and the query cast
    w = lambda k=p, idx=p, ipool=p, H=1, kvdt=1, ks=1.0, idt=1, xs=1.0, q=1, ktf=None: lib.isb_write_cache(  # noqa
        NULL, k, p, idx, p, 4, p, 2, q, H, p, p, kvdt, ks, 1.0, 64, ipool, idt, xs, 8,
        None if ktf is None else ctypes.byref(ktf), None)
    assert w(k=NULL) == -1
    assert w(idx=NULL) == -1 and w(ipool=NULL) == -1            # index vector and pool go together
    assert w(q=0) == -1
    assert w(kvdt=5) == -2 and w(idt=3) == -2
    assert w(ks=0.0) == -1 and w(xs=-1.0) == -1                 # fp8 scales must be positive
    assert w(H=70000) == -3
    assert w(k=ctypes.c_void_p(18)) == -1                       # bf16 pairs are read 4 bytes at a time
    # QK-norm / rope parameters: cos without sin, a rotated width not a multiple of 4, a negative eps
    assert w(ktf=binding.NormRope(rope_cos=16, rope_positions=8, rot_dim=64)) == -1
    assert w(ktf=binding.NormRope(rope_cos=16, rope_sin=32, rope_positions=8, rot_dim=66)) == -3
    assert w(ktf=binding.NormRope(rope_cos=16, rope_sin=32, rope_positions=8, rot_dim=132)) == -3
    assert w(ktf=binding.NormRope(norm_weight=16, eps=-1.0)) == -1
    assert w(ktf=binding.NormRope(rope_cos=16, rope_sin=32, rope_positions=0, rot_dim=64)) == -1
    pq = lambda q=p, H=4, dt=1, nr=None: lib.isb_prepare_query(  # noqa: E731
        NULL, q, H, p, 2, 1, None if nr is None else ctypes.byref(nr), dt, p)
    assert pq(q=NULL) == -1 and pq(H=0) == -1
    assert pq(dt=2) == -2
    assert pq(H=70000) == -3
    assert pq(nr=binding.NormRope(rope_cos=16, rope_sin=32, rope_positions=8, rot_dim=2)) == -3
    # the candidate merge
    assert lib.isb_topk_merge(NULL, NULL, p, 8, p, 1, 1, 1, 16, 4, p) == -1
    assert lib.isb_topk_merge(NULL, p, p, 0, p, 1, 1, 1, 16, 4, p) == -1
    assert lib.isb_topk_merge(NULL, p, p, 1025, p, 1, 1, 1, 16, 4, p) == -3     # too many candidates
    assert lib.isb_topk_merge(NULL, p, p, 8, p, 1, 1, 1, 16, 17, p) == -3       # top_k > max_blocks
    assert lib.isb_quantize_e4m3(NULL, NULL, 4, p) == -1
    assert lib.isb_quantize_e4m3(NULL, p, 0, p) == -1
    # workspace
    need = lib.isb_sparse_pa_workspace_bytes(4, 16, 1, 128, 1)
    assert need > 0
    assert lib.isb_sparse_pa_decode(NULL, p, 0, p, p, 1, 8, 1.0, 1.0, p, 128, p, 4, 1, 16, 1, 128, 0.1,
                                    p, need - 1, p) == -4
    # the allocation-free call refuses partials beyond its 8 MiB array before touching a device:
    # 511 rows of two splits need 511 x 2 x 8320 B
    assert lib.isb_sparse_pa_workspace_bytes(511, 16, 1, 128, 1) == 511 * 2 * 8320 > 8 << 20
    assert lib.isb_sparse_pa_decode_noalloc(NULL, p, 0, p, p, 1, 8, 1.0, 1.0, p, 128, p, 511, 1, 16, 1, 128, 0.1,
                                            p) == -4
    assert lib.isb_sparse_pa_decode_noalloc(NULL, NULL, 0, p, p, 1, 8, 1.0, 1.0, p, 128, p, 4, 1, 16, 1, 128, 0.1,
                                            p) == -1


def test_prefill_argument_checks_return_before_any_launch(lib):
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails its checks first
    # isb_index_score_prefill(stream, q_idx, qdt, H_idx, pool, idt, scale, blocks, bt, stride, R, req, pos, T,
    #                         H_kv, MB, scores)
    sc = lambda q=p, req=p, pos=p, T=8, H=1, R=1, MB=4, stride=4, qdt=0, idt=0: lib.isb_index_score_prefill(  # noqa
        NULL, q, qdt, H, p, idt, 1.0, 8, p, stride, R, req, pos, T, 1, MB, p)
    assert sc(q=NULL) == -1 and sc(req=NULL) == -1 and sc(pos=NULL) == -1
    assert sc(T=0) == -1 and sc(R=0) == -1
    assert sc(qdt=2) == -2 and sc(idt=5) == -2
    assert sc(H=3) == -3                                  # 16 % H_idx
    assert sc(MB=8) == -3                                 # MB > stride
    assert sc(T=65535 * 128 + 1) == -3                    # more than 65535 tiles of 128 rows
    assert sc(T=1 << 28, H=16) == -3                      # rows > 2^31 - 1
    # isb_topk_select_prefill(stream, scores, R, req, pos, T, H_kv, MB, K, topk)
    assert lib.isb_topk_select_prefill(NULL, p, 1, NULL, p, 4, 1, 4, 2, p) == -1
    assert lib.isb_topk_select_prefill(NULL, p, 0, p, p, 4, 1, 4, 2, p) == -1
    assert lib.isb_topk_select_prefill(NULL, p, 1, p, p, 0, 1, 4, 2, p) == -1
    assert lib.isb_topk_select_prefill(NULL, p, 1, p, p, 4, 1, 4, 5, p) == -3    # K > MB
    # isb_emit_sparse_block_table_prefill(stream, topk, bt, stride, R, req, pos, T, H_kv, K, ppb, sbt, sctx)
    assert lib.isb_emit_sparse_block_table_prefill(NULL, p, p, 4, 1, NULL, p, 4, 1, 2, 8, p, p) == -1
    assert lib.isb_emit_sparse_block_table_prefill(NULL, p, p, 4, 1, p, p, 4, 1, 2, 4, p, p) == -3   # ppb 4
    # isb_topk_select_emit_prefill(stream, scores, R, req, pos, T, H_kv, MB, K, bt, stride, ppb, topk, sbt, sctx)
    assert lib.isb_topk_select_emit_prefill(NULL, p, 1, p, NULL, 4, 1, 4, 2, p, 4, 8, p, p, p) == -1
    assert lib.isb_topk_select_emit_prefill(NULL, p, 1, p, p, 4, 1, 8, 2, p, 4, 8, p, p, p) == -3   # MB > stride
    assert lib.isb_topk_select_emit_prefill(NULL, p, 1, p, p, 4, 1, 4, 2, p, 4, 2, p, p, p) == -3   # ppb 2
    # isb_sparse_pa_prefill(stream, q, qdt, kp, vp, kvdt, pages, ks, vs, sbt, stride, sctx, T, Hq, Hkv, hd, sm,
    #                       ws, ws_bytes, out)
    assert lib.isb_sparse_pa_prefill(NULL, p, 0, p, p, 1, 8, 1.0, 1.0, NULL, 8, p, 4, 16, 1, 128, 0.1,
                                     p, 1 << 20, p) == -1
    assert lib.isb_sparse_pa_prefill(NULL, p, 0, p, p, 1, 8, 1.0, 1.0, p, 8, p, 4, 16, 1, 64, 0.1,
                                     p, 1 << 20, p) == -3                                         # head_dim
    need = lib.isb_sparse_pa_workspace_bytes(4, 16, 1, 128, 1)
    assert lib.isb_sparse_pa_prefill(NULL, p, 0, p, p, 1, 8, 1.0, 1.0, p, 128, p, 4, 16, 1, 128, 0.1,
                                     p, need - 1, p) == -4
    # isb_select_attend_prefill(stream, scores, R, req, pos, T, H_kv, MB, K, bt, stride, q, qdt, kp, vp, kvdt,
    #                           pages, ks, vs, Hq, sm, ws, ws_bytes, topk, sbt, sctx, out)
    sa = lambda req=p, R=1, MB=4, K=2, Hq=16: lib.isb_select_attend_prefill(  # noqa: E731
        NULL, p, R, req, p, 4, 1, MB, K, p, 4, p, 0, p, p, 1, 8, 1.0, 1.0, Hq, 0.1, p, 1 << 20, p, p, p, p)
    assert sa(req=NULL) == -1 and sa(R=0) == -1
    assert sa(MB=8) == -3 and sa(K=5) == -3 and sa(Hq=32) == -3


def test_workspace_query(lib):
    # the split-K partials: rows x splits x 16 heads x (128 + 2) floats; the
    # plan's split counts for the five workloads' shapes
    # (none when every row is one split: nothing is published)
    for T, stride, dt, splits in [(128, 128, 1, 2), (4300, 128, 1, 1), (64, 16, 2, 4), (16, 256, 1, 4),
                                  (4, 32, 0, 2)]:
        n = lib.isb_sparse_pa_workspace_bytes(T, 16, 1, stride, dt)
        assert n == (T * splits * 16 * 130 * 4 if splits > 1 else 0), (T, stride, dt)
    assert lib.isb_sparse_pa_workspace_bytes(0, 16, 1, 128, 1) == 0
    assert lib.isb_sparse_pa_workspace_bytes(4, 16, 1, 128, 5) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    with pytest.raises(RuntimeError, match="ROCm GPU"):
        binding.topk_select(torch.zeros(1, 1, 4), torch.ones(1, dtype=torch.int32), 1, 2)


def _fp8_pools(pages, heads=1):
    import torch
    return (torch.zeros(pages, heads * 2048, dtype=torch.uint8), torch.zeros(pages, heads * 2048, dtype=torch.uint8))


def test_binding_refuses_pools_that_do_not_match_before_any_launch(lib):
    # The kernels bound page ids by the K pool's page count and address V with
    # the same id: a V pool shorter than K (the K/V length mismatch vLLM PR
    # 61889 trims), a flat pool or the wrong row size is refused on the host.
    # CPU tensors: every refusal below comes before the device check.
    import torch
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)  # noqa: E731
    q = torch.zeros(2, 16, 128, dtype=torch.bfloat16)
    k, v = _fp8_pools(64)
    for kp, vp in ((k, v[:60]), (k.reshape(-1), v.reshape(-1)), (k[:, :1024], v[:, :1024]),
                   (k.view(torch.int8), v.view(torch.int8))):
        with pytest.raises(ValueError, match="pool"):
            binding.sparse_pa_decode(q, "bf16", kp, vp, "fp8", 1.0, 1.0, i32(2, 128), i32(2), 16, 1, 0.1)
        with pytest.raises(ValueError, match="pool"):
            binding.select_attend(torch.zeros(1, 2, 16), i32(2), 1, 4, i32(2, 16), q, "bf16", kp, vp, "fp8",
                                  1.0, 1.0, 16, 0.1)
        with pytest.raises(ValueError, match="pool"):
            binding.write_cache(torch.zeros(2, 1, 128, dtype=torch.bfloat16),
                                torch.zeros(2, 1, 128, dtype=torch.bfloat16), None, i32(2, 16), i32(2), 1,
                                kp, vp, "fp8", 1.0, 1.0)
    with pytest.raises(ValueError, match="idx_pool"):
        binding.index_score(torch.zeros(2, 1, 128, dtype=torch.bfloat16), "bf16",
                            torch.zeros(8, 8704, dtype=torch.uint8), "fp8", 1.0, i32(2, 8), i32(2), 1, 1, 8)


def test_binding_refuses_wrong_index_and_query_types(lib):
    import torch
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)  # noqa: E731
    k, v = _fp8_pools(64)
    q = torch.zeros(2, 16, 128, dtype=torch.bfloat16)
    # int64 tables and lengths
    with pytest.raises(ValueError, match="int32"):
        binding.sparse_pa_decode(q, "bf16", k, v, "fp8", 1.0, 1.0, torch.zeros(2, 128, dtype=torch.int64),
                                 i32(2), 16, 1, 0.1)
    with pytest.raises(ValueError, match="int32"):
        binding.topk_select(torch.zeros(1, 2, 16), torch.zeros(2, dtype=torch.int64), 1, 4)
    with pytest.raises(ValueError, match="int32"):
        binding.index_score(torch.zeros(2, 1, 128, dtype=torch.bfloat16), "bf16",
                            torch.zeros(8, 16384, dtype=torch.uint8), "fp8", 1.0,
                            torch.zeros(2, 8, dtype=torch.int64), i32(2), 1, 1, 8)
    # a query whose storage does not hold [T, H, 128] elements of its dtype
    with pytest.raises(ValueError, match="q"):
        binding.sparse_pa_decode(torch.zeros(2, 16, 128, dtype=torch.uint8), "bf16", k, v, "fp8", 1.0, 1.0,
                                 i32(2, 128), i32(2), 16, 1, 0.1)
    with pytest.raises(ValueError, match="q_idx"):
        binding.index_score(torch.zeros(2, 1, 64, dtype=torch.bfloat16), "bf16",
                            torch.zeros(8, 16384, dtype=torch.uint8), "fp8", 1.0, i32(2, 8), i32(2), 1, 1, 8)
    with pytest.raises(NotImplementedError):
        binding.sparse_pa_decode(q, "mxfp4", k, v, "fp8", 1.0, 1.0, i32(2, 128), i32(2), 16, 1, 0.1)
    # sparse table rows and lengths must match the query's rows
    with pytest.raises(ValueError, match="sparse_bt"):
        binding.sparse_pa_decode(q, "bf16", k, v, "fp8", 1.0, 1.0, i32(3, 128), i32(2), 16, 1, 0.1)
    with pytest.raises(ValueError, match="sparse_ctx"):
        binding.sparse_pa_decode(q, "bf16", k, v, "fp8", 1.0, 1.0, i32(2, 128), i32(3), 16, 1, 0.1)
    # scores must be fp32 [H_kv, num_reqs * q, MB]
    with pytest.raises(ValueError, match="scores"):
        binding.topk_select(torch.zeros(1, 3, 16), i32(2), 1, 4)
    with pytest.raises(ValueError, match="scores"):
        binding.topk_select(torch.zeros(1, 2, 16, dtype=torch.float64), i32(2), 1, 4)


def test_mfma_overlap_check_reads_register_ranges():
    # The build's assembly check: a destination over a source is caught, an
    # accumulator identical to the destination is not.
    from indexer_selected_block_amd.build import mfma_operand_overlaps
    ok = "  v_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], v[4:7]"
    clash = "  v_mfma_scale_f32_16x16x128_f8f6f4 v[0:3], v[2:9], v[12:19], v[0:3], v20, v21"
    clash_b = "  v_mfma_f32_16x16x16_bf16 a[0:3], v[0:1], a[2:3], a[0:3]"
    assert mfma_operand_overlaps(ok) == []
    assert mfma_operand_overlaps(clash) == [clash.strip()]
    assert mfma_operand_overlaps(clash_b) == [clash_b.strip()]
    assert mfma_operand_overlaps("\n".join([ok, clash])) == [clash.strip()]


def test_bench_refuses_more_than_one_gpu():
    # The path has no multi-GPU part: bench.py --gpus N > 1 says so and exits
    # before touching a device.
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    msg = json.loads(proc.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_bench_counts_each_attended_position_once():
    # The attention's algorithmic bytes: per request and KV head, the union over
    # its query tokens of the positions they attend (a block several tokens
    # select counts once, up to the longest causal reach among them), checked
    # against a set of (head, request, position) built token by token.
    import sys

    import numpy as np
    import torch

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    from indexer_selected_block_amd import workload as wl

    cfg = wl.shrink(wl.CONFIGS["spec_decode"], num_reqs=4, ctx_lo=130, ctx_hi=700, num_pad_reqs=1)
    cfg = wl.replace(cfg, num_kv_heads=2, num_q_heads=16, num_idx_heads=2)
    w = wl.make_workload(cfg, device="cpu")
    rng = np.random.default_rng(3)
    T, ql, K = cfg.num_tokens, cfg.query_len, cfg.top_k
    lens = w.seq_lens.tolist()
    topk = np.full((cfg.num_kv_heads, T, K), -1, dtype=np.int32)
    seen = set()
    for g in range(cfg.num_kv_heads):
        for t in range(T):
            r, i = divmod(t, ql)
            Lt = max(0, lens[r] - (ql - 1 - i))
            nt = -(-Lt // 128)
            if nt == 0:
                continue
            blocks = sorted(set(rng.choice(nt, size=min(K, nt), replace=False).tolist()) | {nt - 1})[:K]
            topk[g, t, :len(blocks)] = blocks
            for b in blocks:
                for pos in range(128 * b, min(128 * b + 128, Lt)):
                    seen.add((g, r, pos))
    import types
    assert bench.distinct_attended_tokens(types.SimpleNamespace(w=w), torch.from_numpy(topk)) == len(seen)
    # a ragged prefill batch, tokens shuffled: the same count from per-token
    # request ids and positions
    b = wl.ragged_batch(w, [min(c, L) for c, L in zip([3, 1, 5, 2, 4], lens)], order="shuffled", seed=4)
    req, pos = b.query_req_id.tolist(), b.query_abs_pos.tolist()
    topk = np.full((cfg.num_kv_heads, b.num_tokens, K), -1, dtype=np.int32)
    seen = set()
    for g in range(cfg.num_kv_heads):
        for t in range(b.num_tokens):
            Lt = pos[t] + 1
            nt = -(-Lt // 128)
            blocks = sorted(set(rng.choice(nt, size=min(K, nt), replace=False).tolist()) | {nt - 1})[:K]
            topk[g, t, :len(blocks)] = blocks
            for bb in blocks:
                for p in range(128 * bb, min(128 * bb + 128, Lt)):
                    seen.add((g, req[t], p))
    L = types.SimpleNamespace(w=w, b=b)
    assert bench.distinct_attended_tokens(L, torch.from_numpy(topk)) == len(seen)


def test_norm_rope_struct_checks_its_tensors():
    # Host logic only: the isb_norm_rope the binding builds, and what it refuses.
    import torch
    w = torch.ones(128)
    cos, sin = torch.zeros(10, 32), torch.zeros(10, 32)
    nr = binding.norm_rope(w, 1e-6, cos, sin, 64, neox=False)
    assert nr.norm_weight == w.data_ptr() and abs(nr.eps - 1e-6) < 1e-12
    assert nr.rope_cos == cos.data_ptr() and nr.rope_sin == sin.data_ptr()
    assert (nr.rope_positions, nr.rot_dim, nr.neox) == (10, 64, 0)
    empty = binding.norm_rope()
    assert not empty.norm_weight and not empty.rope_cos
    with pytest.raises(ValueError):
        binding.norm_rope(torch.ones(64))                      # weight of the wrong width
    with pytest.raises(ValueError):
        binding.norm_rope(w, 1e-6, cos, None, 64)              # cos without sin
    with pytest.raises(ValueError):
        binding.norm_rope(w, 1e-6, cos, sin, 128)              # tables narrower than rot_dim / 2
    with pytest.raises(ValueError):
        binding.norm_rope(w.double())                          # not fp32
