"""Python binding of libisb (ctypes): argument marshalling only.

Each function takes torch tensors that already live on a ROCm device, passes
their device pointers and sizes to the C entry point of the same name
(``isb_<name>``), enqueues on the tensor's current stream and returns the
output tensors.  Every step of the decode runs in the HIP kernels of libisb;
there is no fallback: if the library is not built, or no GPU is present, the
functions raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

BF16, FP8_E4M3, MXFP4 = 0, 1, 2
DTYPE_CODES = {"bf16": BF16, "fp8": FP8_E4M3, "e4m3": FP8_E4M3, "mxfp4": MXFP4}

_STATUS = {
    0: "ok",
    -1: "invalid argument",
    -2: "unsupported dtype",
    -3: "shape mismatch",
    -4: "workspace too small",
    -5: "kernel launch failed",
}

_lib = None


class IsbError(RuntimeError):
    """A libisb call returned an error status."""

    def __init__(self, name: str, status: int):
        self.status = status
        super().__init__(f"isb_{name}: {_STATUS.get(status, 'unknown error')} (status {status})")


def _exc(name: str, status: int) -> Exception:
    err = IsbError(name, status)
    if status in (-1, -3, -4):
        return ValueError(str(err))
    if status == -2:
        return NotImplementedError(str(err))
    return err


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

class NormRope(ctypes.Structure):
    """isb_norm_rope: the optional QK-norm and rope of the fused writer."""
    _fields_ = [("norm_weight", ctypes.c_void_p), ("eps", ctypes.c_float), ("rope_cos", ctypes.c_void_p),
                ("rope_sin", ctypes.c_void_p), ("rope_positions", ctypes.c_int64), ("rot_dim", ctypes.c_int),
                ("neox", ctypes.c_int)]


def norm_rope(norm_weight=None, eps=0.0, rope_cos=None, rope_sin=None, rot_dim=0, neox=True):
    """An isb_norm_rope from fp32 device tensors: norm_weight [128], rope_cos /
    rope_sin [positions, rot_dim / 2] (None: that part is not applied).  The
    tensors must outlive the calls that use it."""
    nr = NormRope()
    if norm_weight is not None:
        if norm_weight.dtype != torch.float32 or norm_weight.shape != (128,) or not norm_weight.is_contiguous():
            raise ValueError("norm_weight is fp32 [128]")
        nr.norm_weight, nr.eps = norm_weight.data_ptr(), float(eps)
    if rope_cos is not None or rope_sin is not None:
        for t in (rope_cos, rope_sin):
            if t is None or t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != rot_dim // 2 or \
                    not t.is_contiguous():
                raise ValueError("rope_cos / rope_sin are fp32 [positions, rot_dim / 2]")
        if rope_cos.shape != rope_sin.shape:
            raise ValueError("rope_cos and rope_sin differ in shape")
        nr.rope_cos, nr.rope_sin = rope_cos.data_ptr(), rope_sin.data_ptr()
        nr.rope_positions, nr.rot_dim, nr.neox = rope_cos.shape[0], int(rot_dim), int(bool(neox))
    return nr


_NR = ctypes.POINTER(NormRope)

_SIGNATURES = {
    "isb_version": ([], _I),
    "isb_strerror": ([_I], ctypes.c_char_p),
    "isb_index_score": ([_P, _P, _I, _I, _P, _I, _F, _I64, _P, _I, _P, _I, _I, _I, _I, _P], _I),
    "isb_topk_select": ([_P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "isb_emit_sparse_block_table": ([_P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P], _I),
    "isb_topk_select_emit": ([_P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P], _I),
    "isb_select_attend": ([_P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _P, _I, _I64, _F, _F, _I, _F,
                           _P, _SZ, _P, _P, _P, _P], _I),
    "isb_sparse_pa_workspace_bytes": ([_I, _I, _I, _I, _I], _SZ),
    "isb_sparse_pa_decode": ([_P, _P, _I, _P, _P, _I, _I64, _F, _F, _P, _I, _P, _I, _I, _I, _I, _I,
                              _F, _P, _SZ, _P], _I),
    "isb_sparse_pa_decode_noalloc": ([_P, _P, _I, _P, _P, _I, _I64, _F, _F, _P, _I, _P, _I, _I, _I, _I, _I,
                                      _F, _P], _I),
    "isb_write_cache": ([_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _P, _I, _F, _F, _I64, _P, _I, _F, _I64,
                         _NR, _NR], _I),
    "isb_prepare_query": ([_P, _P, _I, _P, _I, _I, _NR, _I, _P], _I),
    "isb_topk_merge": ([_P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P], _I),
    "isb_quantize_e4m3": ([_P, _P, _I64, _P], _I),
    "isb_index_score_prefill": ([_P, _P, _I, _I, _P, _I, _F, _I64, _P, _I, _I, _P, _P, _I, _I, _I, _P], _I),
    "isb_topk_select_prefill": ([_P, _P, _I, _P, _P, _I, _I, _I, _I, _P], _I),
    "isb_emit_sparse_block_table_prefill": ([_P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "isb_topk_select_emit_prefill": ([_P, _P, _I, _P, _P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P], _I),
    "isb_sparse_pa_prefill": ([_P, _P, _I, _P, _P, _I, _I64, _F, _F, _P, _I, _P, _I, _I, _I, _I, _F, _P, _SZ,
                               _P], _I),
    "isb_select_attend_prefill": ([_P, _P, _I, _P, _P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _P, _I, _I64, _F, _F,
                                   _I, _F, _P, _SZ, _P, _P, _P, _P], _I),
}
EXPORTED = tuple(_SIGNATURES)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open libisb.so and declare its entry points (no GPU needed)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path == LIB_PATH:
        _lib = lib
    return lib


def _call(name: str, *args) -> None:
    status = getattr(load_library(), "isb_" + name)(*args)
    if status != 0:
        raise _exc(name, status)


def _dev(*tensors: torch.Tensor) -> torch.device:
    dev = tensors[0].device
    if dev.type != "cuda":
        raise RuntimeError("libisb runs on a ROCm GPU: tensors must be on a cuda device")
    for t in tensors:
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _code(dtype) -> int:
    return DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)


# Bytes of one page: a K or V page of one KV head (16 tokens bf16 / fp8, 128
# tokens MXFP4) and an index page (128 tokens).
KV_PAGE_BYTES = {BF16: 4096, FP8_E4M3: 2048, MXFP4: 8704}
IDX_PAGE_BYTES = {BF16: 32768, FP8_E4M3: 16384, MXFP4: 8704}


def _check_kv_pools(k_pool, v_pool, kv_dtype, num_kv_heads) -> int:
    """K and V pools: uint8 [pages, num_kv_heads * page bytes], the same shape
    (one page id addresses both, so the kernels bound V by K's page count);
    returns the page count."""
    code = _code(kv_dtype)
    if code not in KV_PAGE_BYTES:
        raise NotImplementedError(f"K/V dtype {kv_dtype!r} is not bf16, fp8 or mxfp4")
    row = num_kv_heads * KV_PAGE_BYTES[code]
    for name, pool in (("k_pool", k_pool), ("v_pool", v_pool)):
        if pool.dtype != torch.uint8 or pool.dim() != 2 or pool.shape[1] != row:
            raise ValueError(f"{name} must be uint8 [pages, {row}] (num_kv_heads x page bytes), "
                             f"got {pool.dtype} {tuple(pool.shape)}")
    if v_pool.shape != k_pool.shape:
        raise ValueError(f"k_pool {tuple(k_pool.shape)} and v_pool {tuple(v_pool.shape)} must have the same "
                         f"pages: one page id addresses both")
    return k_pool.shape[0]


def _check_idx_pool(idx_pool, idx_dtype) -> int:
    """Index pool: uint8 [blocks, index page bytes]; returns the block count."""
    code = _code(idx_dtype)
    if code not in IDX_PAGE_BYTES:
        raise NotImplementedError(f"index dtype {idx_dtype!r} is not bf16, fp8 or mxfp4")
    row = IDX_PAGE_BYTES[code]
    if idx_pool.dtype != torch.uint8 or idx_pool.dim() != 2 or idx_pool.shape[1] != row:
        raise ValueError(f"idx_pool must be uint8 [blocks, {row}], got {idx_pool.dtype} {tuple(idx_pool.shape)}")
    return idx_pool.shape[0]


def _check_int32(**tensors) -> None:
    for name, t in tensors.items():
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32, got {t.dtype}")


def _check_query(name, q, q_dtype, tokens, heads) -> None:
    """A query [tokens, heads, 128] stored as bf16 (2 bytes an element) or e4m3
    (1 byte): any torch dtype whose storage has exactly that many bytes."""
    code = _code(q_dtype)
    if code not in (BF16, FP8_E4M3):
        raise NotImplementedError(f"{name} dtype {q_dtype!r} is not bf16 or e4m3")
    want = tokens * heads * 128 * (2 if code == BF16 else 1)
    if q.dim() < 2 or q.shape[0] != tokens or q.shape[1] != heads or q.numel() * q.element_size() != want:
        raise ValueError(f"{name} must hold [{tokens}, {heads}, 128] {'bf16' if code == BF16 else 'e4m3'} "
                         f"elements, got {q.dtype} {tuple(q.shape)}")


def _check_shape(name, t, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def version() -> int:
    return int(load_library().isb_version())


def strerror(status: int) -> str:
    return load_library().isb_strerror(int(status)).decode()


def index_score(q_idx, q_idx_dtype, idx_pool, idx_dtype, idx_scale, block_table, seq_lens,
                decode_query_len, num_kv_heads, max_blocks, scores=None):
    """Block scores [num_kv_heads, T, max_blocks] fp32 (see isb_index_score)."""
    T, H_idx = q_idx.shape[0], q_idx.shape[1]
    _check_idx_pool(idx_pool, idx_dtype)
    _check_int32(block_table=block_table, seq_lens=seq_lens)
    R = seq_lens.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != R or seq_lens.dim() != 1:
        raise ValueError("block_table is [num_reqs, stride] and seq_lens [num_reqs]")
    if T != R * decode_query_len:
        raise ValueError(f"q_idx has {T} tokens, expected num_reqs * decode_query_len = {R * decode_query_len}")
    _check_query("q_idx", q_idx, q_idx_dtype, T, H_idx)
    dev = _dev(q_idx, idx_pool, block_table, seq_lens)
    if scores is None:
        scores = torch.empty((num_kv_heads, T, max_blocks), dtype=torch.float32, device=dev)
    _dev(scores)
    if scores.dtype != torch.float32:
        raise ValueError("scores must be float32")
    _check_shape("scores", scores, (num_kv_heads, T, max_blocks))
    _call("index_score", _stream(dev), q_idx.data_ptr(), _code(q_idx_dtype), H_idx,
          idx_pool.data_ptr(), _code(idx_dtype), float(idx_scale), idx_pool.shape[0],
          block_table.data_ptr(), block_table.shape[1], seq_lens.data_ptr(), seq_lens.shape[0],
          decode_query_len, num_kv_heads, max_blocks, scores.data_ptr())
    return scores


def _check_scores(scores, seq_lens, decode_query_len):
    """scores fp32 [H_kv, T, max_blocks] with T = num_reqs * decode_query_len; seq_lens int32."""
    _check_int32(seq_lens=seq_lens)
    if scores.dtype != torch.float32 or scores.dim() != 3:
        raise ValueError("scores must be float32 [num_kv_heads, T, max_blocks]")
    if scores.shape[1] != seq_lens.shape[0] * decode_query_len:
        raise ValueError("scores has T != num_reqs * decode_query_len rows")
    return scores.shape


def _check_table(block_table, seq_lens):
    _check_int32(block_table=block_table)
    if block_table.dim() != 2 or block_table.shape[0] != seq_lens.shape[0]:
        raise ValueError("block_table must be int32 [num_reqs, stride]")


def topk_select(scores, seq_lens, decode_query_len, top_k, topk_idx=None):
    """Selected blocks [num_kv_heads, T, top_k] int32 (see isb_topk_select)."""
    H_kv, T, MB = _check_scores(scores, seq_lens, decode_query_len)
    dev = _dev(scores, seq_lens)
    if topk_idx is None:
        topk_idx = torch.empty((H_kv, T, top_k), dtype=torch.int32, device=dev)
    _dev(topk_idx)
    _check_int32(topk_idx=topk_idx)
    _check_shape("topk_idx", topk_idx, (H_kv, T, top_k))
    _call("topk_select", _stream(dev), scores.data_ptr(), seq_lens.data_ptr(), seq_lens.shape[0],
          decode_query_len, H_kv, MB, top_k, topk_idx.data_ptr())
    return topk_idx


def emit_sparse_block_table(topk_idx, block_table, seq_lens, decode_query_len, pages_per_block,
                            sparse_bt=None, sparse_ctx=None):
    """(sparse_bt [T*H_kv, K*ppb], sparse_ctx [T*H_kv]) int32 (see isb_emit_sparse_block_table)."""
    _check_int32(topk_idx=topk_idx, seq_lens=seq_lens)
    _check_table(block_table, seq_lens)
    H_kv, T, K = topk_idx.shape
    if T != seq_lens.shape[0] * decode_query_len:
        raise ValueError("topk_idx has T != num_reqs * decode_query_len rows")
    dev = _dev(topk_idx, block_table, seq_lens)
    if sparse_bt is None:
        sparse_bt = torch.empty((T * H_kv, K * pages_per_block), dtype=torch.int32, device=dev)
    if sparse_ctx is None:
        sparse_ctx = torch.empty((T * H_kv,), dtype=torch.int32, device=dev)
    _dev(sparse_bt, sparse_ctx)
    _check_int32(sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    _check_shape("sparse_bt", sparse_bt, (T * H_kv, K * pages_per_block))
    _check_shape("sparse_ctx", sparse_ctx, (T * H_kv,))
    _call("emit_sparse_block_table", _stream(dev), topk_idx.data_ptr(), block_table.data_ptr(),
          block_table.shape[1], seq_lens.data_ptr(), seq_lens.shape[0], decode_query_len, H_kv, K,
          pages_per_block, sparse_bt.data_ptr(), sparse_ctx.data_ptr())
    return sparse_bt, sparse_ctx


def topk_select_emit(scores, seq_lens, decode_query_len, top_k, block_table, pages_per_block,
                     topk_idx=None, sparse_bt=None, sparse_ctx=None):
    """(topk_idx, sparse_bt, sparse_ctx) in one launch (see isb_topk_select_emit)."""
    H_kv, T, MB = _check_scores(scores, seq_lens, decode_query_len)
    _check_table(block_table, seq_lens)
    dev = _dev(scores, seq_lens, block_table)
    if topk_idx is None:
        topk_idx = torch.empty((H_kv, T, top_k), dtype=torch.int32, device=dev)
    if sparse_bt is None:
        sparse_bt = torch.empty((T * H_kv, top_k * pages_per_block), dtype=torch.int32, device=dev)
    if sparse_ctx is None:
        sparse_ctx = torch.empty((T * H_kv,), dtype=torch.int32, device=dev)
    _dev(topk_idx, sparse_bt, sparse_ctx)
    _check_int32(topk_idx=topk_idx, sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    _check_shape("topk_idx", topk_idx, (H_kv, T, top_k))
    _check_shape("sparse_bt", sparse_bt, (T * H_kv, top_k * pages_per_block))
    _check_shape("sparse_ctx", sparse_ctx, (T * H_kv,))
    _call("topk_select_emit", _stream(dev), scores.data_ptr(), seq_lens.data_ptr(), seq_lens.shape[0],
          decode_query_len, H_kv, MB, top_k, block_table.data_ptr(), block_table.shape[1],
          pages_per_block, topk_idx.data_ptr(), sparse_bt.data_ptr(), sparse_ctx.data_ptr())
    return topk_idx, sparse_bt, sparse_ctx


def topk_merge(cand_scores, cand_ids, seq_lens, decode_query_len, top_k, max_blocks, topk_idx=None):
    """Selections [H_kv, T, top_k] int32 from candidates [H_kv, T, C] (see isb_topk_merge)."""
    if cand_scores.shape != cand_ids.shape or cand_scores.dim() != 3:
        raise ValueError("cand_scores and cand_ids are [H_kv, T, C]")
    if cand_scores.dtype != torch.float32 or cand_ids.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("cand_scores fp32, cand_ids and seq_lens int32")
    H_kv, T, C = cand_ids.shape
    if T != seq_lens.shape[0] * decode_query_len:
        raise ValueError("T must be num_reqs * query_len")
    dev = _dev(cand_scores, cand_ids, seq_lens)
    if topk_idx is None:
        topk_idx = torch.empty((H_kv, T, top_k), dtype=torch.int32, device=dev)
    _dev(topk_idx)
    _call("topk_merge", _stream(dev), cand_scores.data_ptr(), cand_ids.data_ptr(), C, seq_lens.data_ptr(),
          seq_lens.shape[0], decode_query_len, H_kv, max_blocks, top_k, topk_idx.data_ptr())
    return topk_idx


def sparse_pa_workspace_bytes(num_tokens, num_q_heads, num_kv_heads, sparse_bt_stride, kv_dtype) -> int:
    return int(load_library().isb_sparse_pa_workspace_bytes(
        num_tokens, num_q_heads, num_kv_heads, sparse_bt_stride, _code(kv_dtype)))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """An attention workspace in its initial state: zero-filled (every split
    partial slot free).  Every completed call leaves it so."""
    return torch.zeros((max(int(nbytes), 16),), dtype=torch.uint8, device=device)


def _check_out(out, T, num_q_heads):
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16")
    _check_shape("out", out, (T, num_q_heads, 128))


def sparse_pa_decode(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale, v_scale, sparse_bt, sparse_ctx,
                     num_q_heads, num_kv_heads, sm_scale, out=None, workspace=None, decode_query_len=1):
    """Attention output [T, num_q_heads, 128] bf16 (see isb_sparse_pa_decode;
    decode_query_len: query tokens per request, which only decides how pages
    are read)."""
    T = q.shape[0]
    num_pages = _check_kv_pools(k_pool, v_pool, kv_dtype, num_kv_heads)
    _check_query("q", q, q_dtype, T, num_q_heads)
    _check_int32(sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    if sparse_bt.dim() != 2 or sparse_bt.shape[0] != T * num_kv_heads:
        raise ValueError(f"sparse_bt must be int32 [{T * num_kv_heads}, stride]")
    _check_shape("sparse_ctx", sparse_ctx, (T * num_kv_heads,))
    dev = _dev(q, k_pool, v_pool, sparse_bt, sparse_ctx)
    stride = sparse_bt.shape[1]
    need = sparse_pa_workspace_bytes(T, num_q_heads, num_kv_heads, stride, kv_dtype)
    if workspace is None:
        workspace = new_workspace(need, dev)
    if out is None:
        out = torch.empty((T, num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    _dev(out, workspace)
    _check_out(out, T, num_q_heads)
    _call("sparse_pa_decode", _stream(dev), q.data_ptr(), _code(q_dtype), k_pool.data_ptr(),
          v_pool.data_ptr(), _code(kv_dtype), num_pages, float(k_scale), float(v_scale),
          sparse_bt.data_ptr(), stride, sparse_ctx.data_ptr(), T, int(decode_query_len), num_q_heads,
          num_kv_heads, 128,
          float(sm_scale), workspace.data_ptr(), workspace.numel(), out.data_ptr())
    return out


def sparse_pa_decode_noalloc(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale, v_scale, sparse_bt, sparse_ctx,
                             num_q_heads, num_kv_heads, sm_scale, out, decode_query_len=1):
    """sparse_pa_decode into a caller-owned ``out`` with no workspace: the
    split partials go to the library's own device array (see
    isb_sparse_pa_decode_noalloc).  Allocates nothing."""
    T = q.shape[0]
    num_pages = _check_kv_pools(k_pool, v_pool, kv_dtype, num_kv_heads)
    _check_query("q", q, q_dtype, T, num_q_heads)
    _check_int32(sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    if sparse_bt.dim() != 2 or sparse_bt.shape[0] != T * num_kv_heads:
        raise ValueError(f"sparse_bt must be int32 [{T * num_kv_heads}, stride]")
    _check_shape("sparse_ctx", sparse_ctx, (T * num_kv_heads,))
    _check_out(out, T, num_q_heads)
    dev = _dev(q, k_pool, v_pool, sparse_bt, sparse_ctx, out)
    _call("sparse_pa_decode_noalloc", _stream(dev), q.data_ptr(), _code(q_dtype), k_pool.data_ptr(),
          v_pool.data_ptr(), _code(kv_dtype), num_pages, float(k_scale), float(v_scale), sparse_bt.data_ptr(),
          sparse_bt.shape[1], sparse_ctx.data_ptr(), T, int(decode_query_len), num_q_heads, num_kv_heads, 128,
          float(sm_scale), out.data_ptr())
    return out


def select_attend(scores, seq_lens, decode_query_len, top_k, block_table, q, q_dtype, k_pool, v_pool,
                  kv_dtype, k_scale, v_scale, num_q_heads, sm_scale, topk_idx=None, sparse_bt=None,
                  sparse_ctx=None, out=None, workspace=None):
    """(topk_idx, sparse_bt, sparse_ctx, out): top-k, emit and attention (see isb_select_attend)."""
    H_kv, T, MB = _check_scores(scores, seq_lens, decode_query_len)
    _check_table(block_table, seq_lens)
    num_pages = _check_kv_pools(k_pool, v_pool, kv_dtype, H_kv)
    _check_query("q", q, q_dtype, T, num_q_heads)
    dev = _dev(scores, seq_lens, block_table, q, k_pool, v_pool)
    ppb = 1 if _code(kv_dtype) == DTYPE_CODES["mxfp4"] else 8
    if topk_idx is None:
        topk_idx = torch.empty((H_kv, T, top_k), dtype=torch.int32, device=dev)
    if sparse_bt is None:
        sparse_bt = torch.empty((T * H_kv, top_k * ppb), dtype=torch.int32, device=dev)
    if sparse_ctx is None:
        sparse_ctx = torch.empty((T * H_kv,), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((T, num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    need = sparse_pa_workspace_bytes(T, num_q_heads, H_kv, top_k * ppb, kv_dtype)
    if workspace is None:
        workspace = new_workspace(need, dev)
    _dev(topk_idx, sparse_bt, sparse_ctx, out, workspace)
    _check_int32(topk_idx=topk_idx, sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    _check_shape("topk_idx", topk_idx, (H_kv, T, top_k))
    _check_shape("sparse_bt", sparse_bt, (T * H_kv, top_k * ppb))
    _check_shape("sparse_ctx", sparse_ctx, (T * H_kv,))
    _check_out(out, T, num_q_heads)
    _call("select_attend", _stream(dev), scores.data_ptr(), seq_lens.data_ptr(), seq_lens.shape[0],
          decode_query_len, H_kv, MB, top_k, block_table.data_ptr(), block_table.shape[1], q.data_ptr(),
          _code(q_dtype), k_pool.data_ptr(), v_pool.data_ptr(), _code(kv_dtype), num_pages,
          float(k_scale), float(v_scale), num_q_heads, float(sm_scale), workspace.data_ptr(),
          workspace.numel(), topk_idx.data_ptr(), sparse_bt.data_ptr(), sparse_ctx.data_ptr(), out.data_ptr())
    return topk_idx, sparse_bt, sparse_ctx, out


# ---------------------------------------------------------------- prefill batches
def _check_tokens(query_req_id, query_abs_pos, block_table) -> int:
    """Per-token request ids and positions, int32 [T]; block_table int32
    [num_reqs, stride].  Returns T."""
    _check_int32(query_req_id=query_req_id, query_abs_pos=query_abs_pos, block_table=block_table)
    if query_req_id.dim() != 1 or query_abs_pos.shape != query_req_id.shape:
        raise ValueError("query_req_id and query_abs_pos must be int32 [num_tokens]")
    if block_table.dim() != 2:
        raise ValueError("block_table must be int32 [num_reqs, stride]")
    return int(query_req_id.shape[0])


def _check_prefill_scores(scores, T):
    if scores.dtype != torch.float32 or scores.dim() != 3 or scores.shape[1] != T:
        raise ValueError(f"scores must be float32 [num_kv_heads, {T}, max_blocks]")
    return scores.shape


def index_score_prefill(q_idx, q_idx_dtype, idx_pool, idx_dtype, idx_scale, block_table, query_req_id,
                        query_abs_pos, num_kv_heads, max_blocks, scores=None):
    """Block scores [num_kv_heads, T, max_blocks] fp32 of a prefill batch (see
    isb_index_score_prefill)."""
    T = _check_tokens(query_req_id, query_abs_pos, block_table)
    H_idx = q_idx.shape[1]
    _check_idx_pool(idx_pool, idx_dtype)
    _check_query("q_idx", q_idx, q_idx_dtype, T, H_idx)
    dev = _dev(q_idx, idx_pool, block_table, query_req_id, query_abs_pos)
    if scores is None:
        scores = torch.empty((num_kv_heads, T, max_blocks), dtype=torch.float32, device=dev)
    _dev(scores)
    if scores.dtype != torch.float32:
        raise ValueError("scores must be float32")
    _check_shape("scores", scores, (num_kv_heads, T, max_blocks))
    _call("index_score_prefill", _stream(dev), q_idx.data_ptr(), _code(q_idx_dtype), H_idx,
          idx_pool.data_ptr(), _code(idx_dtype), float(idx_scale), idx_pool.shape[0], block_table.data_ptr(),
          block_table.shape[1], block_table.shape[0], query_req_id.data_ptr(), query_abs_pos.data_ptr(), T,
          num_kv_heads, max_blocks, scores.data_ptr())
    return scores


def topk_select_prefill(scores, num_reqs, query_req_id, query_abs_pos, top_k, topk_idx=None):
    """Selections [num_kv_heads, T, top_k] int32 of a prefill batch (see
    isb_topk_select_prefill)."""
    _check_int32(query_req_id=query_req_id, query_abs_pos=query_abs_pos)
    T = int(query_req_id.shape[0])
    H_kv, _, MB = _check_prefill_scores(scores, T)
    dev = _dev(scores, query_req_id, query_abs_pos)
    if topk_idx is None:
        topk_idx = torch.empty((H_kv, T, top_k), dtype=torch.int32, device=dev)
    _dev(topk_idx)
    _check_int32(topk_idx=topk_idx)
    _check_shape("topk_idx", topk_idx, (H_kv, T, top_k))
    _call("topk_select_prefill", _stream(dev), scores.data_ptr(), int(num_reqs), query_req_id.data_ptr(),
          query_abs_pos.data_ptr(), T, H_kv, MB, top_k, topk_idx.data_ptr())
    return topk_idx


def emit_sparse_block_table_prefill(topk_idx, block_table, query_req_id, query_abs_pos, pages_per_block,
                                    sparse_bt=None, sparse_ctx=None):
    """(sparse_bt [T*H_kv, K*ppb], sparse_ctx [T*H_kv]) int32 of a prefill batch
    (see isb_emit_sparse_block_table_prefill)."""
    T = _check_tokens(query_req_id, query_abs_pos, block_table)
    _check_int32(topk_idx=topk_idx)
    H_kv, Tk, K = topk_idx.shape
    if Tk != T:
        raise ValueError("topk_idx must have one row per token")
    dev = _dev(topk_idx, block_table, query_req_id, query_abs_pos)
    if sparse_bt is None:
        sparse_bt = torch.empty((T * H_kv, K * pages_per_block), dtype=torch.int32, device=dev)
    if sparse_ctx is None:
        sparse_ctx = torch.empty((T * H_kv,), dtype=torch.int32, device=dev)
    _dev(sparse_bt, sparse_ctx)
    _check_int32(sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    _check_shape("sparse_bt", sparse_bt, (T * H_kv, K * pages_per_block))
    _check_shape("sparse_ctx", sparse_ctx, (T * H_kv,))
    _call("emit_sparse_block_table_prefill", _stream(dev), topk_idx.data_ptr(), block_table.data_ptr(),
          block_table.shape[1], block_table.shape[0], query_req_id.data_ptr(), query_abs_pos.data_ptr(), T,
          H_kv, K, pages_per_block, sparse_bt.data_ptr(), sparse_ctx.data_ptr())
    return sparse_bt, sparse_ctx


def topk_select_emit_prefill(scores, query_req_id, query_abs_pos, top_k, block_table, pages_per_block,
                             topk_idx=None, sparse_bt=None, sparse_ctx=None):
    """(topk_idx, sparse_bt, sparse_ctx) of a prefill batch in one launch (see
    isb_topk_select_emit_prefill)."""
    T = _check_tokens(query_req_id, query_abs_pos, block_table)
    H_kv, _, MB = _check_prefill_scores(scores, T)
    dev = _dev(scores, block_table, query_req_id, query_abs_pos)
    if topk_idx is None:
        topk_idx = torch.empty((H_kv, T, top_k), dtype=torch.int32, device=dev)
    if sparse_bt is None:
        sparse_bt = torch.empty((T * H_kv, top_k * pages_per_block), dtype=torch.int32, device=dev)
    if sparse_ctx is None:
        sparse_ctx = torch.empty((T * H_kv,), dtype=torch.int32, device=dev)
    _dev(topk_idx, sparse_bt, sparse_ctx)
    _check_int32(topk_idx=topk_idx, sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    _check_shape("topk_idx", topk_idx, (H_kv, T, top_k))
    _check_shape("sparse_bt", sparse_bt, (T * H_kv, top_k * pages_per_block))
    _check_shape("sparse_ctx", sparse_ctx, (T * H_kv,))
    _call("topk_select_emit_prefill", _stream(dev), scores.data_ptr(), block_table.shape[0],
          query_req_id.data_ptr(), query_abs_pos.data_ptr(), T, H_kv, MB, top_k, block_table.data_ptr(),
          block_table.shape[1], pages_per_block, topk_idx.data_ptr(), sparse_bt.data_ptr(), sparse_ctx.data_ptr())
    return topk_idx, sparse_bt, sparse_ctx


def sparse_pa_prefill(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale, v_scale, sparse_bt, sparse_ctx,
                      num_q_heads, num_kv_heads, sm_scale, out=None, workspace=None):
    """Attention output [T, num_q_heads, 128] bf16 for the rows of a prefill
    batch (see isb_sparse_pa_prefill)."""
    T = q.shape[0]
    num_pages = _check_kv_pools(k_pool, v_pool, kv_dtype, num_kv_heads)
    _check_query("q", q, q_dtype, T, num_q_heads)
    _check_int32(sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    if sparse_bt.dim() != 2 or sparse_bt.shape[0] != T * num_kv_heads:
        raise ValueError(f"sparse_bt must be int32 [{T * num_kv_heads}, stride]")
    _check_shape("sparse_ctx", sparse_ctx, (T * num_kv_heads,))
    dev = _dev(q, k_pool, v_pool, sparse_bt, sparse_ctx)
    stride = sparse_bt.shape[1]
    need = sparse_pa_workspace_bytes(T, num_q_heads, num_kv_heads, stride, kv_dtype)
    if workspace is None:
        workspace = new_workspace(need, dev)
    if out is None:
        out = torch.empty((T, num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    _dev(out, workspace)
    _check_out(out, T, num_q_heads)
    _call("sparse_pa_prefill", _stream(dev), q.data_ptr(), _code(q_dtype), k_pool.data_ptr(),
          v_pool.data_ptr(), _code(kv_dtype), num_pages, float(k_scale), float(v_scale), sparse_bt.data_ptr(),
          stride, sparse_ctx.data_ptr(), T, num_q_heads, num_kv_heads, 128, float(sm_scale),
          workspace.data_ptr(), workspace.numel(), out.data_ptr())
    return out


def select_attend_prefill(scores, query_req_id, query_abs_pos, top_k, block_table, q, q_dtype, k_pool, v_pool,
                          kv_dtype, k_scale, v_scale, num_q_heads, sm_scale, topk_idx=None, sparse_bt=None,
                          sparse_ctx=None, out=None, workspace=None):
    """(topk_idx, sparse_bt, sparse_ctx, out) of a prefill batch (see
    isb_select_attend_prefill)."""
    T = _check_tokens(query_req_id, query_abs_pos, block_table)
    H_kv, _, MB = _check_prefill_scores(scores, T)
    num_pages = _check_kv_pools(k_pool, v_pool, kv_dtype, H_kv)
    _check_query("q", q, q_dtype, T, num_q_heads)
    dev = _dev(scores, block_table, query_req_id, query_abs_pos, q, k_pool, v_pool)
    ppb = 1 if _code(kv_dtype) == DTYPE_CODES["mxfp4"] else 8
    if topk_idx is None:
        topk_idx = torch.empty((H_kv, T, top_k), dtype=torch.int32, device=dev)
    if sparse_bt is None:
        sparse_bt = torch.empty((T * H_kv, top_k * ppb), dtype=torch.int32, device=dev)
    if sparse_ctx is None:
        sparse_ctx = torch.empty((T * H_kv,), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((T, num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    need = sparse_pa_workspace_bytes(T, num_q_heads, H_kv, top_k * ppb, kv_dtype)
    if workspace is None:
        workspace = new_workspace(need, dev)
    _dev(topk_idx, sparse_bt, sparse_ctx, out, workspace)
    _check_int32(topk_idx=topk_idx, sparse_bt=sparse_bt, sparse_ctx=sparse_ctx)
    _check_shape("topk_idx", topk_idx, (H_kv, T, top_k))
    _check_shape("sparse_bt", sparse_bt, (T * H_kv, top_k * ppb))
    _check_shape("sparse_ctx", sparse_ctx, (T * H_kv,))
    _check_out(out, T, num_q_heads)
    _call("select_attend_prefill", _stream(dev), scores.data_ptr(), block_table.shape[0], query_req_id.data_ptr(),
          query_abs_pos.data_ptr(), T, H_kv, MB, top_k, block_table.data_ptr(), block_table.shape[1], q.data_ptr(),
          _code(q_dtype), k_pool.data_ptr(), v_pool.data_ptr(), _code(kv_dtype), num_pages, float(k_scale),
          float(v_scale), num_q_heads, float(sm_scale), workspace.data_ptr(), workspace.numel(),
          topk_idx.data_ptr(), sparse_bt.data_ptr(), sparse_ctx.data_ptr(), out.data_ptr())
    return topk_idx, sparse_bt, sparse_ctx, out


def write_cache(k_new, v_new, idx_new, block_table, seq_lens, decode_query_len, k_pool, v_pool, kv_dtype,
                k_scale, v_scale, idx_pool=None, idx_dtype="bf16", idx_scale=1.0, k_norm_rope=None,
                idx_norm_rope=None):
    """Stores the step's new K, V (and index keys, unless idx_new is None) into
    the pools, in place, K and index keys after their optional QK-norm / rope
    (``norm_rope(...)`` structures; see isb_write_cache)."""
    _call("write_cache", *_write_cache_args(k_new, v_new, idx_new, block_table, seq_lens, decode_query_len,
                                            k_pool, v_pool, kv_dtype, k_scale, v_scale, idx_pool, idx_dtype,
                                            idx_scale, k_norm_rope, idx_norm_rope))


def write_cache_launcher(*args, **kwargs):
    """write_cache's arguments checked once: returns a callable that enqueues
    the same write again (same tensors, same stream) with no further checks."""
    a = _write_cache_args(*args, **kwargs)
    return lambda: _call("write_cache", *a)


def _ref(nr):
    return None if nr is None else ctypes.byref(nr)


def _write_cache_args(k_new, v_new, idx_new, block_table, seq_lens, decode_query_len, k_pool, v_pool, kv_dtype,
                      k_scale, v_scale, idx_pool=None, idx_dtype="bf16", idx_scale=1.0, k_norm_rope=None,
                      idx_norm_rope=None):
    if (idx_new is None) != (idx_pool is None):
        raise ValueError("idx_new and idx_pool go together")
    R, H_kv = seq_lens.shape[0], k_new.shape[1]
    T = R * decode_query_len
    if k_new.shape != (T, H_kv, 128) or v_new.shape != (T, H_kv, 128) or \
            (idx_new is not None and idx_new.shape != (T, 128)):
        raise ValueError("k_new, v_new [T, H_kv, 128] and idx_new [T, 128] with T = num_reqs * query_len")
    for t in (k_new, v_new) + (() if idx_new is None else (idx_new,)):
        if t.dtype != torch.bfloat16:
            raise ValueError("new keys and values are bf16")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or block_table.shape[0] != R:
        raise ValueError("block_table [num_reqs, stride] and seq_lens [num_reqs] are int32")
    _check_kv_pools(k_pool, v_pool, kv_dtype, H_kv)
    if idx_pool is not None:
        _check_idx_pool(idx_pool, idx_dtype)
    dev = _dev(k_new, v_new, block_table, seq_lens, k_pool, v_pool,
               *(() if idx_new is None else (idx_new, idx_pool)))
    return (_stream(dev), k_new.data_ptr(), v_new.data_ptr(),
            None if idx_new is None else idx_new.data_ptr(), block_table.data_ptr(), block_table.shape[1],
            seq_lens.data_ptr(), R, decode_query_len, H_kv, k_pool.data_ptr(),
            v_pool.data_ptr(), _code(kv_dtype), float(k_scale), float(v_scale), k_pool.shape[0],
            None if idx_pool is None else idx_pool.data_ptr(), _code(idx_dtype), float(idx_scale),
            0 if idx_pool is None else idx_pool.shape[0], _ref(k_norm_rope), _ref(idx_norm_rope))


def quantize_e4m3(x, out=None):
    """uint8 e4m3fn codes of a bf16 tensor, unit scale (see isb_quantize_e4m3)."""
    dev = _dev(x)
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    _dev(out)
    if out.numel() != x.numel():
        raise ValueError("out must have x's size")
    if x.numel():
        _call("quantize_e4m3", _stream(dev), x.data_ptr(), x.numel(), out.data_ptr())
    return out


def prepare_query(q, seq_lens, decode_query_len, norm_rope=None, out_dtype="e4m3", out=None):
    """q [T, H, 128] bf16 after its optional QK-norm / rope, as e4m3 codes
    (uint8) or bf16 (see isb_prepare_query)."""
    dev = _dev(q, seq_lens)
    T, H = q.shape[0], q.shape[1]
    if q.dtype != torch.bfloat16 or q.shape[2] != 128 or T != seq_lens.shape[0] * decode_query_len:
        raise ValueError("q is bf16 [num_reqs * query_len, H, 128]")
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens is int32")
    code = _code(out_dtype)
    if out is None:
        out = torch.empty((T, H, 128), dtype=torch.bfloat16 if code == BF16 else torch.uint8, device=dev)
    _dev(out)
    if out.numel() != q.numel() or out.element_size() != (2 if code == BF16 else 1):
        raise ValueError("out must match q's shape in the output dtype")
    _call("prepare_query", _stream(dev), q.data_ptr(), H, seq_lens.data_ptr(), seq_lens.shape[0],
          decode_query_len, _ref(norm_rope), code, out.data_ptr())
    return out


class DecodeLayer:
    """One decode layer over a workload, with persistent outputs: index_score,
    then select_attend (top-k, the sparse table and the attention, in one launch
    where the shapes allow it).

    Buffers are allocated once at construction (torch, on the workload's
    device); ``run()`` only enqueues the launches, so it can be timed or
    captured."""

    def __init__(self, w):
        cfg = w.cfg
        self.w = w
        dev = w.q.device
        T = cfg.num_tokens
        self.scores = torch.empty((cfg.num_kv_heads, T, cfg.max_blocks), dtype=torch.float32, device=dev)
        self.topk = torch.empty((cfg.num_kv_heads, T, cfg.top_k), dtype=torch.int32, device=dev)
        ppb = cfg.pages_per_block
        self.sparse_bt = torch.empty((T * cfg.num_kv_heads, cfg.top_k * ppb), dtype=torch.int32, device=dev)
        self.sparse_ctx = torch.empty((T * cfg.num_kv_heads,), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, cfg.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
        need = sparse_pa_workspace_bytes(T, cfg.num_q_heads, cfg.num_kv_heads, cfg.top_k * ppb, cfg.kv_dtype)
        self.workspace = new_workspace(need, dev)

    def run(self):
        w, cfg = self.w, self.w.cfg
        index_score(w.q_idx, cfg.qidx_dtype, w.idx_pool, cfg.idx_dtype, w.idx_scale, w.block_table,
                    w.seq_lens, cfg.query_len, cfg.num_kv_heads, cfg.max_blocks, scores=self.scores)
        select_attend(self.scores, w.seq_lens, cfg.query_len, cfg.top_k, w.block_table, w.q, cfg.q_dtype,
                      w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, cfg.num_q_heads, w.sm_scale,
                      topk_idx=self.topk, sparse_bt=self.sparse_bt, sparse_ctx=self.sparse_ctx, out=self.out,
                      workspace=self.workspace)
        return self.out


class PrefillLayer:
    """One sparse prefill layer over a ragged batch (per-token request ids and
    positions) of a workload's requests: index_score_prefill, then
    select_attend_prefill, with persistent outputs, as DecodeLayer."""

    def __init__(self, w, batch):
        cfg = w.cfg
        self.w, self.b = w, batch
        dev = w.q.device
        T = batch.num_tokens
        self.scores = torch.empty((cfg.num_kv_heads, T, cfg.max_blocks), dtype=torch.float32, device=dev)
        self.topk = torch.empty((cfg.num_kv_heads, T, cfg.top_k), dtype=torch.int32, device=dev)
        ppb = cfg.pages_per_block
        self.sparse_bt = torch.empty((T * cfg.num_kv_heads, cfg.top_k * ppb), dtype=torch.int32, device=dev)
        self.sparse_ctx = torch.empty((T * cfg.num_kv_heads,), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, cfg.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
        need = sparse_pa_workspace_bytes(T, cfg.num_q_heads, cfg.num_kv_heads, cfg.top_k * ppb, cfg.kv_dtype)
        self.workspace = new_workspace(need, dev)

    def run(self):
        w, b, cfg = self.w, self.b, self.w.cfg
        index_score_prefill(b.q_idx, cfg.qidx_dtype, w.idx_pool, cfg.idx_dtype, w.idx_scale, w.block_table,
                            b.query_req_id, b.query_abs_pos, cfg.num_kv_heads, cfg.max_blocks, scores=self.scores)
        select_attend_prefill(self.scores, b.query_req_id, b.query_abs_pos, cfg.top_k, w.block_table, b.q,
                              cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, cfg.num_q_heads,
                              w.sm_scale, topk_idx=self.topk, sparse_bt=self.sparse_bt, sparse_ctx=self.sparse_ctx,
                              out=self.out, workspace=self.workspace)
        return self.out


# C names, for callers that prefer them.
isb_index_score = index_score
isb_topk_select = topk_select
isb_emit_sparse_block_table = emit_sparse_block_table
isb_topk_select_emit = topk_select_emit
isb_select_attend = select_attend
isb_sparse_pa_decode = sparse_pa_decode
isb_sparse_pa_decode_noalloc = sparse_pa_decode_noalloc
isb_sparse_pa_workspace_bytes = sparse_pa_workspace_bytes
isb_index_score_prefill = index_score_prefill
isb_topk_select_prefill = topk_select_prefill
isb_emit_sparse_block_table_prefill = emit_sparse_block_table_prefill
isb_topk_select_emit_prefill = topk_select_emit_prefill
isb_sparse_pa_prefill = sparse_pa_prefill
isb_select_attend_prefill = select_attend_prefill
