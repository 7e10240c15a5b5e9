"""Seeded synthetic inputs for one layer of indexed block-sparse paged-attention decode.

This module only draws random numbers, rounds them into the storage formats the
caches use and lays them out in pool pages.  It performs no step of the decode
(no scoring, selection, table emission or attention); the GPU path and the CPU
oracle both read what it produces, each with code of its own.

Pool layout (the contract every reader follows)
-----------------------------------------------
A request's token at absolute position ``p`` lives in the 128-token block
``block_table[r][p // 128]`` at slot ``p % 128``.

* Index cache, one page per 128-token block (page id == block id):
  - bf16:  128 tokens x 128 dims, 32768 B: eight 16-token tiles, each laid out
           like a 16-token K page (``k_page16_bytes``);
  - fp8:   the same with e4m3 elements, 16384 B, times one per-tensor scale
           ``idx_scale``;
  - MXFP4: 8704 B = 128 x 64 B of e2m1 data (token j at byte 64 j, dim d in
           byte d // 2, low nibble for even d) followed by 128 x 4 B of e8m0
           scales (token j at byte 8192 + 4 j, scale s covering dims 32 s ..
           32 s + 31).  This is the page of ROCm/ATOM PR 2962 ("MXFP4 index
           cache and MXFP4 KV cache", Summary and the layout commit message).
* K/V caches in bf16 / fp8 use 16-token pages, 8 per block (pages_per_block 8):
  block ``b``'s pages are ``8 b .. 8 b + 7``; page ``8 b + s // 16`` holds
  slot ``s``.  Pages are laid out in 16-byte chunks in the order the
  attention kernel's lanes read them (see ``k_page16_bytes`` /
  ``v_page16_bytes``).  fp8 values carry per-tensor ``k_scale`` /
  ``v_scale``.  One page id addresses the K page and the V page alike.
* K/V caches in MXFP4 use one 8704 B page per block (pages_per_block 1), the
  same page format as the MXFP4 index cache, for K and for V.
* A K/V page id holds one page per KV head: the pools are
  ``[num_pages][H_kv][page bytes]`` (the index cache has a single key per
  token, shared by every index head, so it has no head dimension).

Slots a request has not written (past its length) and every page no request
uses hold poison (NaN in every format), and unused block-table entries point
at a dedicated all-poison block, so a read outside the selection shows up as
NaN rather than as a plausible number or a memory fault.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

HEAD_DIM = 128
BLOCK_TOKENS = 128
PAGE16_TOKENS = 16
MXFP4_PAGE_BYTES = BLOCK_TOKENS * HEAD_DIM // 2 + BLOCK_TOKENS * HEAD_DIM // 32  # 8704

POOL_DTYPES = ("bf16", "fp8", "mxfp4")
QUERY_DTYPES = ("bf16", "e4m3")

# Poison bytes: bf16 quiet NaN, e4m3 NaN (0x7F), MXFP4 page of 0xFF (e8m0 0xFF is NaN).
_BF16_NAN_BITS = 0x7FC0
_E4M3_NAN = 0x7F
_MX_POISON = 0xFF

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Config:
    name: str
    num_reqs: int          # live requests
    query_len: int         # decode_query_len q
    ctx_lo: int            # live context lengths ~ U{ctx_lo .. ctx_hi}
    ctx_hi: int
    num_pad_reqs: int      # extra requests of length 0 at seeded slots
    num_kv_heads: int
    num_q_heads: int
    num_idx_heads: int
    top_k: int             # blocks kept per row
    idx_dtype: str         # index cache: bf16 | fp8 | mxfp4
    kv_dtype: str          # K/V cache:   bf16 | fp8 | mxfp4
    q_dtype: str           # main query:  bf16 | e4m3
    qidx_dtype: str        # index query: bf16 | e4m3
    pool_blocks: int       # 128-token blocks in the pools (plus one poison block)
    key_dist: str          # normal | student_t3 | mx_uniform
    seed: int
    description: str = ""
    head_dim: int = HEAD_DIM

    @property
    def total_reqs(self) -> int:
        return self.num_reqs + self.num_pad_reqs

    @property
    def num_tokens(self) -> int:
        return self.total_reqs * self.query_len

    @property
    def max_blocks(self) -> int:
        return -(-self.ctx_hi // BLOCK_TOKENS)

    @property
    def pages_per_block(self) -> int:
        return 1 if self.kv_dtype == "mxfp4" else BLOCK_TOKENS // PAGE16_TOKENS

    @property
    def page_tokens(self) -> int:
        return BLOCK_TOKENS // self.pages_per_block


# The five workloads.  Shapes, dtypes and value distributions follow the
# configurations the method is measured on; where those are silent the plainest
# reading is taken (index query bf16 unless e4m3 is named, H_idx = 1 per KV head,
# "65536-page pool" counted in 128-token blocks because 16-token pages could not
# hold the batch).
CONFIGS: dict[str, Config] = {
    "tiny_bf16": Config(
        "tiny_bf16", num_reqs=4, query_len=1, ctx_lo=1024, ctx_hi=1024, num_pad_reqs=0,
        num_kv_heads=1, num_q_heads=8, num_idx_heads=1, top_k=4,
        idx_dtype="bf16", kv_dtype="bf16", q_dtype="bf16", qidx_dtype="bf16",
        pool_blocks=64, key_dist="normal", seed=1,
        description="4 requests x 1 token, 1024-token contexts, bf16 K/V and index, top-k 4"),
    "fp8_decode": Config(
        "fp8_decode", num_reqs=128, query_len=1, ctx_lo=16384, ctx_hi=65536, num_pad_reqs=0,
        num_kv_heads=1, num_q_heads=16, num_idx_heads=1, top_k=16,
        idx_dtype="fp8", kv_dtype="fp8", q_dtype="bf16", qidx_dtype="bf16",
        pool_blocks=65536, key_dist="normal", seed=2,
        description="128 requests x 1 token, contexts U{16384..65536}, fp8 K/V and index, top-k 16"),
    "spec_decode": Config(
        "spec_decode", num_reqs=1024, query_len=4, ctx_lo=4096, ctx_hi=32768, num_pad_reqs=51,
        num_kv_heads=1, num_q_heads=16, num_idx_heads=1, top_k=16,
        idx_dtype="fp8", kv_dtype="fp8", q_dtype="bf16", qidx_dtype="bf16",
        pool_blocks=262144, key_dist="normal", seed=3,
        description="1024 requests x 4 tokens + 51 pad requests, contexts U{4096..32768}, fp8, top-k 16"),
    "mxfp4": Config(
        "mxfp4", num_reqs=64, query_len=1, ctx_lo=131072, ctx_hi=131072, num_pad_reqs=0,
        num_kv_heads=1, num_q_heads=16, num_idx_heads=4, top_k=16,
        idx_dtype="mxfp4", kv_dtype="mxfp4", q_dtype="e4m3", qidx_dtype="e4m3",
        pool_blocks=65536, key_dist="mx_uniform", seed=4,
        description="64 requests x 1 token, 131072-token contexts, MXFP4 K/V and index, 4 index heads"),
    "long_context": Config(
        "long_context", num_reqs=8, query_len=2, ctx_lo=1048576, ctx_hi=1048576, num_pad_reqs=0,
        num_kv_heads=1, num_q_heads=16, num_idx_heads=1, top_k=32,
        idx_dtype="mxfp4", kv_dtype="fp8", q_dtype="bf16", qidx_dtype="e4m3",
        pool_blocks=890768 // 8, key_dist="student_t3", seed=5,
        description="8 requests x 2 tokens, 1048576-token contexts, fp8 K/V, MXFP4 index, top-k 32"),
    # Chunked prefill: the last 512 tokens of each request are the query chunk,
    # each token with its own causal top-k (the decode formulas with
    # decode_query_len = 512); otherwise the fp8 decode workload's setup.
    "prefill": Config(
        "prefill", num_reqs=4, query_len=512, ctx_lo=16384, ctx_hi=65536, num_pad_reqs=0,
        num_kv_heads=1, num_q_heads=16, num_idx_heads=1, top_k=16,
        idx_dtype="fp8", kv_dtype="fp8", q_dtype="bf16", qidx_dtype="bf16",
        pool_blocks=4 * 512 + 64, key_dist="normal", seed=6,
        description="4 requests x 512-token prefill chunks, contexts U{16384..65536}, fp8 K/V and index, "
                    "top-k 16 per token"),
    # The same chunks with the index query cast to unit-scale e4m3 (the index
    # query form of the MXFP4 path, here against fp8 keys): the scorer then
    # multiplies keys as stored on the fp8 MFMA.
    "prefill_e4m3q": Config(
        "prefill_e4m3q", num_reqs=4, query_len=512, ctx_lo=16384, ctx_hi=65536, num_pad_reqs=0,
        num_kv_heads=1, num_q_heads=16, num_idx_heads=1, top_k=16,
        idx_dtype="fp8", kv_dtype="fp8", q_dtype="bf16", qidx_dtype="e4m3",
        pool_blocks=4 * 512 + 64, key_dist="normal", seed=6,
        description="4 requests x 512-token prefill chunks, contexts U{16384..65536}, fp8 K/V and index, "
                    "e4m3 index query, top-k 16 per token"),
}


# Ragged prefill batches: each request contributes the last chunk_lens[r]
# positions of its context as query tokens, each token carrying its own
# request id and absolute position (the prefill call's query_req_id /
# query_abs_pos).  The setup is the prefill workload's (fp8 K/V and index,
# contexts U{16384..65536}, top-k 16 per token) with six requests whose chunks
# run from a single token to 1024 tokens.
RAGGED_CHUNKS: dict[str, tuple[int, ...]] = {
    "prefill_ragged": (512, 1, 300, 77, 1024, 133),
}


def ragged_config(name: str) -> Config:
    """The request-level setup of a ragged prefill batch (query_len unused: 1)."""
    chunks = RAGGED_CHUNKS[name]
    base = CONFIGS["prefill"]
    return replace(base, name=name, num_reqs=len(chunks), query_len=1,
                   pool_blocks=len(chunks) * base.max_blocks + 64, seed=7,
                   description=f"{len(chunks)} requests with prefill chunks of "
                               f"{'/'.join(map(str, chunks))} tokens ({sum(chunks)} in all), contexts "
                               "U{16384..65536}, fp8 K/V and index, top-k 16 per token")


@dataclass
class RaggedBatch:
    query_req_id: torch.Tensor   # int32 [T]: the token's row of the block table
    query_abs_pos: torch.Tensor  # int32 [T]: its 0-based position in the request
    q: torch.Tensor              # uint8 [T, H_q, 128 * qbytes]
    q_idx: torch.Tensor          # uint8 [T, H_idx, 128 * qbytes]

    @property
    def num_tokens(self) -> int:
        return int(self.query_req_id.shape[0])

    def to(self, device) -> "RaggedBatch":
        return RaggedBatch(*(t.to(device) for t in (self.query_req_id, self.query_abs_pos, self.q,
                                                      self.q_idx)))


def ragged_batch(w: "Workload", chunk_lens, order: str = "grouped", seed: int = 0) -> RaggedBatch:
    """Query tokens of a ragged prefill over the requests of ``w``: request r
    gives its last chunk_lens[r] positions (0 = none).  ``order``: "grouped"
    (request by request, positions ascending: a prefill batch as a scheduler
    lays it out) or "shuffled" (a seeded permutation of the same tokens).
    Fresh seeded queries of the workload's query dtypes."""
    cfg = w.cfg
    lens = w.seq_lens.cpu().to(torch.int64)
    chunks = torch.as_tensor(list(chunk_lens), dtype=torch.int64)
    if chunks.shape[0] != lens.shape[0] or bool((chunks < 0).any()) or bool((chunks > lens).any()):
        raise ValueError("one chunk length a request, each within the request's length")
    req = torch.repeat_interleave(torch.arange(lens.shape[0]), chunks)
    first = torch.cumsum(chunks, 0) - chunks
    pos = lens[req] - chunks[req] + (torch.arange(req.shape[0]) - first[req])
    if order == "shuffled":
        perm = torch.randperm(req.shape[0], generator=torch.Generator().manual_seed(seed * 31 + 5))
        req, pos = req[perm], pos[perm]
    elif order != "grouped":
        raise ValueError(order)
    T = int(req.shape[0])
    streams = _Streams(cfg.seed * 1009 + seed, torch.device("cpu"))
    q = _query(cfg, streams, _T_Q, (T, cfg.num_q_heads, cfg.head_dim), cfg.q_dtype)
    q_idx = _query(cfg, streams, _T_QIDX, (T, cfg.num_idx_heads, cfg.head_dim), cfg.qidx_dtype)
    dev = w.seq_lens.device
    return RaggedBatch(req.to(torch.int32).to(dev), pos.to(torch.int32).to(dev), q.to(dev), q_idx.to(dev))


def shrink(cfg: Config, num_reqs: int, ctx_lo: int, ctx_hi: int, num_pad_reqs: int | None = None,
           pool_blocks: int | None = None, top_k: int | None = None) -> Config:
    """A smaller workload with the same dtypes, heads and query length."""
    nb = -(-ctx_hi // BLOCK_TOKENS)
    pad = cfg.num_pad_reqs if num_pad_reqs is None else num_pad_reqs
    need = num_reqs * nb
    return replace(cfg, name=f"{cfg.name}_small", num_reqs=num_reqs, ctx_lo=ctx_lo,
                   ctx_hi=ctx_hi, num_pad_reqs=pad,
                   pool_blocks=pool_blocks if pool_blocks is not None else max(need + need // 4, 8),
                   top_k=cfg.top_k if top_k is None else top_k)


@dataclass
class Workload:
    cfg: Config
    seq_lens: torch.Tensor      # int32 [R]
    block_table: torch.Tensor   # int32 [R, max_blocks]
    q: torch.Tensor             # uint8 [T, H_q, 128 * qbytes]
    q_idx: torch.Tensor         # uint8 [T, H_idx, 128 * qbytes]
    idx_pool: torch.Tensor      # uint8 [pool_blocks + 1, idx page bytes]
    k_pool: torch.Tensor        # uint8 [num_pages, H_kv * page bytes]
    v_pool: torch.Tensor        # uint8 [num_pages, H_kv * page bytes]
    idx_scale: float
    k_scale: float
    v_scale: float
    sm_scale: float
    extras: dict = field(default_factory=dict)

    @property
    def num_pages(self) -> int:
        return self.k_pool.shape[0]

    def to(self, device) -> "Workload":
        mv = lambda t: t.to(device)  # noqa: E731
        return replace(self, seq_lens=mv(self.seq_lens), block_table=mv(self.block_table),
                       q=mv(self.q), q_idx=mv(self.q_idx), idx_pool=mv(self.idx_pool),
                       k_pool=mv(self.k_pool), v_pool=mv(self.v_pool))


def idx_page_bytes(dtype: str) -> int:
    return {"bf16": BLOCK_TOKENS * HEAD_DIM * 2, "fp8": BLOCK_TOKENS * HEAD_DIM,
            "mxfp4": MXFP4_PAGE_BYTES}[dtype]


def kv_page_bytes(dtype: str) -> int:
    return {"bf16": PAGE16_TOKENS * HEAD_DIM * 2, "fp8": PAGE16_TOKENS * HEAD_DIM,
            "mxfp4": MXFP4_PAGE_BYTES}[dtype]


# ---------------------------------------------------------------- rounding helpers
def _to_bf16_bytes(x: torch.Tensor) -> torch.Tensor:
    """float -> bf16 (round to nearest even), returned as raw little-endian bytes."""
    return x.to(torch.bfloat16).view(torch.uint8)


def _to_e4m3_bytes(x: torch.Tensor) -> torch.Tensor:
    """float -> e4m3fn, saturating at +-448, round to nearest even, as raw bytes."""
    return x.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


# e2m1 magnitudes by code 0..7 and the round-to-nearest-even decision points.
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _to_e2m1_codes(x: torch.Tensor) -> torch.Tensor:
    """float (already divided by its block scale) -> 4-bit e2m1 codes, RNE, saturating at 6."""
    a = x.abs()
    # Midpoints between neighbouring magnitudes; a tie goes to the even code
    # (the one with mantissa bit 0), i.e. ties at 0.25, 1.25, 2.5 go down and
    # 0.75, 1.75, 3.5, 5 go up.
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], device=x.device, dtype=x.dtype)
    up_on_tie = torch.tensor([False, True, False, True, False, True, True], device=x.device)
    code = torch.zeros_like(a, dtype=torch.int64)
    for i in range(7):
        code += ((a > mids[i]) | ((a == mids[i]) & up_on_tie[i])).to(torch.int64)
    sign = (x < 0) | ((x == 0) & torch.signbit(x))
    return (code | (sign.to(torch.int64) << 3)).to(torch.uint8)


def _mx_quantize(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """OCP MX quantisation of [..., 128] floats: per 32 elements a shared exponent
    floor(log2(amax)) - 2 (e2m1's largest exponent), elements rounded to e2m1.
    Returns (codes uint8 [..., 128], e8m0 scale bytes uint8 [..., 4])."""
    g = x.reshape(*x.shape[:-1], 4, 32)
    amax = g.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.full_like(amax, -127.0))
    e = e.clamp(-127, 127)
    scale = torch.exp2(e)
    codes = _to_e2m1_codes((g / scale.unsqueeze(-1)).reshape(x.shape))
    return codes, (e + 127).to(torch.uint8)


def _pack_mxfp4_page(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """codes uint8 [n, 128 tok, 128 dim] (4-bit values) + scales [n, 128, 4] -> [n, 8704] bytes."""
    n = codes.shape[0]
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    data = (lo | (hi << 4)).reshape(n, BLOCK_TOKENS * HEAD_DIM // 2)
    return torch.cat([data, scales.reshape(n, BLOCK_TOKENS * 4)], dim=1)


# ---------------------------------------------------------------- 16-token page layout
def k_page16_bytes(x: torch.Tensor) -> torch.Tensor:
    """K values as bytes [n, 16 tok, 128 dim, esize] -> pages [n, 16 * 128 * esize].

    Chunk h (16 bytes) of lane l = 16 g + c sits at byte 1024 h + 16 l and holds
    key c's dims 32 g + (16 / esize) h .. (+ 16 / esize - 1): dim d of key c
    lives at byte 1024 ((d mod 32) div dpc) + 256 (d div 32) + 16 c + esize (d mod dpc),
    dpc = 16 / esize dims per chunk."""
    n, esz = x.shape[0], x.shape[-1]
    dpc = 16 // esz
    y = x.reshape(n, PAGE16_TOKENS, 4, 32 // dpc, 16)      # [n, c, g, h, chunk bytes]
    return y.permute(0, 3, 2, 1, 4).reshape(n, -1)


def v_page16_bytes(x: torch.Tensor) -> torch.Tensor:
    """V values as bytes [n, 16 tok, 128 dim, esize] -> pages [n, 16 * 128 * esize].

    Chunk h of lane l = 16 g + c sits at byte 1024 h + 16 l and holds, for the
    dim tiles dt = tpc h .. tpc h + tpc - 1 (tpc = 4 / esize), keys 4 g .. 4 g + 3
    of dim 16 dt + c: key t = 4 g + e, dim 16 dt + c lives at byte
    1024 (dt div tpc) + 16 (16 g + c) + 4 esize (dt mod tpc) + esize e."""
    n, esz = x.shape[0], x.shape[-1]
    tpc = 4 // esz
    y = x.reshape(n, 4, 4, 8 // tpc, tpc, 16, esz)          # [n, g, e, h, q, c, byte]
    return y.permute(0, 3, 1, 5, 4, 2, 6).reshape(n, -1)


# ---------------------------------------------------------------- generation
class _Streams:
    """Independent, reproducible torch generators keyed by (config seed, purpose, chunk)."""

    def __init__(self, seed: int, device):
        self.seed = seed
        self.device = torch.device(device)

    def gen(self, *key: int) -> torch.Generator:
        g = torch.Generator(device=self.device)
        s = self.seed
        for k in key:
            s = (s * 1000003 + k + 1) % (2**63 - 1)
        g.manual_seed(s)
        return g


_T_KEYS, _T_K, _T_V, _T_Q, _T_QIDX = 1, 2, 3, 4, 5


def _draw(cfg: Config, streams: _Streams, tensor_id: int, chunk: int, shape, dist: str) -> torch.Tensor:
    g = streams.gen(tensor_id, chunk)
    dev = streams.device
    if dist == "normal":
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
    if dist == "student_t3":
        z = torch.randn((4, *shape), generator=g, device=dev, dtype=torch.float32)
        chi2 = (z[1] ** 2 + z[2] ** 2 + z[3] ** 2)
        return z[0] / torch.sqrt(chi2.clamp_min(1e-30) / 3.0)
    raise ValueError(dist)


def _lengths(cfg: Config, streams: _Streams) -> torch.Tensor:
    g = torch.Generator().manual_seed(cfg.seed * 7919 + 17)
    live = torch.randint(cfg.ctx_lo, cfg.ctx_hi + 1, (cfg.num_reqs,), generator=g, dtype=torch.int64)
    lens = torch.zeros(cfg.total_reqs, dtype=torch.int64)
    if cfg.num_pad_reqs:
        pad_slots = torch.randperm(cfg.total_reqs, generator=g)[: cfg.num_pad_reqs]
        mask = torch.ones(cfg.total_reqs, dtype=torch.bool)
        mask[pad_slots] = False
        lens[mask] = live
    else:
        lens[:] = live
    return lens


def make_workload(cfg: Config, device="cpu", chunk_blocks: int = 2048) -> Workload:
    """Build the pools, tables and queries of ``cfg`` on ``device`` (seeded, reproducible)."""
    dev = torch.device(device)
    streams = _Streams(cfg.seed, dev)
    lens = _lengths(cfg, streams)
    R, MB, ppb = cfg.total_reqs, cfg.max_blocks, cfg.pages_per_block
    nblk = (lens + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    used = int(nblk.sum())
    if used > cfg.pool_blocks:
        raise ValueError(f"{cfg.name}: batch needs {used} blocks, pool has {cfg.pool_blocks}")
    poison_block = cfg.pool_blocks
    g = torch.Generator().manual_seed(cfg.seed * 104729 + 3)
    ids = torch.randperm(cfg.pool_blocks, generator=g)[:used]
    bt = torch.full((R, MB), poison_block, dtype=torch.int64)
    # per used block: request, block index within the request, valid slots
    req_of = torch.repeat_interleave(torch.arange(R), nblk)
    first = torch.cumsum(nblk, 0) - nblk
    bidx = torch.arange(used) - first[req_of]
    bt[req_of, bidx] = ids
    valid = (lens[req_of] - bidx * BLOCK_TOKENS).clamp(max=BLOCK_TOKENS)

    nb_pool = cfg.pool_blocks + 1
    idx_pool = torch.empty((nb_pool, idx_page_bytes(cfg.idx_dtype)), dtype=torch.uint8, device=dev)
    kv_block_bytes = kv_page_bytes(cfg.kv_dtype) * ppb * cfg.num_kv_heads
    k_pool = torch.empty((nb_pool, kv_block_bytes), dtype=torch.uint8, device=dev)
    v_pool = torch.empty((nb_pool, kv_block_bytes), dtype=torch.uint8, device=dev)
    _fill_poison(idx_pool, cfg.idx_dtype)
    _fill_poison(k_pool, cfg.kv_dtype)
    _fill_poison(v_pool, cfg.kv_dtype)

    ids_d = ids.to(dev)
    valid_d = valid.to(dev)
    # Keys (index and K) follow the config's key distribution; V is N(0,1) except
    # on the MXFP4 workload, where every cache draws codes and exponents uniformly.
    key_dist_kv = cfg.key_dist
    # fp8 per-tensor scales: amax / 448 over the values actually written.
    idx_scale = _write_cache(cfg, streams, _T_KEYS, idx_pool, cfg.idx_dtype, "idx", ids_d, valid_d,
                             cfg.key_dist, chunk_blocks, 1, 1)
    k_scale = _write_cache(cfg, streams, _T_K, k_pool, cfg.kv_dtype, "k", ids_d, valid_d,
                           key_dist_kv, chunk_blocks, ppb, cfg.num_kv_heads)
    v_scale = _write_cache(cfg, streams, _T_V, v_pool, cfg.kv_dtype, "v", ids_d, valid_d,
                           "normal" if cfg.key_dist != "mx_uniform" else "mx_uniform", chunk_blocks,
                           ppb, cfg.num_kv_heads)

    T = cfg.num_tokens
    q = _query(cfg, streams, _T_Q, (T, cfg.num_q_heads, cfg.head_dim), cfg.q_dtype)
    q_idx = _query(cfg, streams, _T_QIDX, (T, cfg.num_idx_heads, cfg.head_dim), cfg.qidx_dtype)

    page_bytes = kv_page_bytes(cfg.kv_dtype)
    return Workload(
        cfg=cfg,
        seq_lens=lens.to(torch.int32).to(dev),
        block_table=bt.to(torch.int32).to(dev),
        q=q, q_idx=q_idx, idx_pool=idx_pool,
        k_pool=k_pool.view(nb_pool * ppb, cfg.num_kv_heads * page_bytes),
        v_pool=v_pool.view(nb_pool * ppb, cfg.num_kv_heads * page_bytes),
        idx_scale=idx_scale, k_scale=k_scale, v_scale=v_scale,
        sm_scale=1.0 / math.sqrt(cfg.head_dim),
    )


def _fill_poison(pool: torch.Tensor, dtype: str) -> None:
    if dtype == "bf16":
        pool.view(torch.int16).fill_(_BF16_NAN_BITS)
    elif dtype == "fp8":
        pool.fill_(_E4M3_NAN)
    else:
        pool.fill_(_MX_POISON)


def _query(cfg: Config, streams: _Streams, tid: int, shape, dtype: str) -> torch.Tensor:
    x = _draw(cfg, streams, tid, 0, shape, "normal")
    if dtype == "bf16":
        return _to_bf16_bytes(x).reshape(shape[0], shape[1], -1).contiguous()
    return _to_e4m3_bytes(x).reshape(shape[0], shape[1], -1).contiguous()


def _chunks(n: int, size: int):
    for s in range(0, n, size):
        yield s // size, s, min(n, s + size)


def _write_cache(cfg, streams, tid, pool, dtype, which, ids, valid, dist, chunk_blocks, ppb,
                 heads) -> float:
    """Fill the used blocks of one cache; returns the per-tensor scale (1.0 unless fp8).

    ``pool`` is [blocks, ppb * heads * page bytes]: per block, ``ppb`` pages,
    each holding one page per head."""
    n = ids.shape[0]
    dev = streams.device
    slot = torch.arange(BLOCK_TOKENS, device=dev)
    pv = pool.view(pool.shape[0], ppb, heads, -1)

    def put(s, e, h, page):
        pv[ids[s:e], :, h, :] = page.reshape(e - s, ppb, -1)

    if dtype == "mxfp4" and dist == "mx_uniform":
        # e2m1 codes uniform over all 16 codes; e8m0 exponents uniform in [-4, 4].
        for h in range(heads):
            for c, s, e in _chunks(n, chunk_blocks):
                g = streams.gen(tid + 100 * h, c)
                codes = torch.randint(0, 16, (e - s, BLOCK_TOKENS, HEAD_DIM), generator=g,
                                      device=dev, dtype=torch.int64).to(torch.uint8)
                sc = torch.randint(127 - 4, 127 + 5, (e - s, BLOCK_TOKENS, 4), generator=g,
                                   device=dev, dtype=torch.int64).to(torch.uint8)
                page = _pack_mxfp4_page(codes, sc)
                _poison_tail(page, valid[s:e], slot, dtype, which)
                put(s, e, h, page)
        return 1.0

    scale = 1.0
    if dtype == "fp8":
        amax = torch.zeros((), device=dev)
        for h in range(heads):
            for c, s, e in _chunks(n, chunk_blocks):
                x = _draw(cfg, streams, tid + 100 * h, c, (e - s, BLOCK_TOKENS, HEAD_DIM), dist)
                m = (slot[None, :] < valid[s:e, None]).unsqueeze(-1)
                amax = torch.maximum(amax, (x.abs() * m).amax())
        scale = float(amax) / E4M3_MAX if float(amax) > 0 else 1.0
    for h in range(heads):
        for c, s, e in _chunks(n, chunk_blocks):
            x = _draw(cfg, streams, tid + 100 * h, c, (e - s, BLOCK_TOKENS, HEAD_DIM), dist)
            nb = e - s
            if dtype == "mxfp4":
                codes, sc = _mx_quantize(x)
                page = _pack_mxfp4_page(codes, sc)
                _poison_tail(page, valid[s:e], slot, dtype, which)
                put(s, e, h, page)
                continue
            if dtype == "bf16":
                vals = _to_bf16_bytes(x).reshape(nb, BLOCK_TOKENS, HEAD_DIM, 2)
            else:
                vals = _to_e4m3_bytes(x / scale).reshape(nb, BLOCK_TOKENS, HEAD_DIM, 1)
            # poison the unwritten slots in token order, then lay out the pages
            bad = slot[None, :] >= valid[s:e, None]
            pz = torch.tensor([0xC0, 0x7F] if dtype == "bf16" else [_E4M3_NAN],
                              dtype=torch.uint8, device=dev)
            vals = torch.where(bad[:, :, None, None], pz, vals)
            if which == "idx":
                tiles = vals.reshape(nb * 8, PAGE16_TOKENS, HEAD_DIM, vals.shape[-1])
                page = k_page16_bytes(tiles).reshape(nb, -1)
            else:
                pages16 = vals.reshape(nb * 8, PAGE16_TOKENS, HEAD_DIM, vals.shape[-1])
                lay = k_page16_bytes if which == "k" else v_page16_bytes
                page = lay(pages16).reshape(nb, -1)
            put(s, e, h, page)
    return scale


def _poison_tail(page: torch.Tensor, valid: torch.Tensor, slot: torch.Tensor, dtype: str, which: str) -> None:
    """Overwrite the slots past each block's written length with poison
    (MXFP4 pages, which are token-major)."""
    nb = page.shape[0]
    bad = slot[None, :] >= valid[:, None]            # [nb, 128]
    if not bool(bad.any()):
        return
    if dtype == "mxfp4":
        data = page[:, : BLOCK_TOKENS * 64].view(nb, BLOCK_TOKENS, 64)
        scl = page[:, BLOCK_TOKENS * 64:].view(nb, BLOCK_TOKENS, 4)
        data.masked_fill_(bad.unsqueeze(-1), _MX_POISON)
        scl.masked_fill_(bad.unsqueeze(-1), _MX_POISON)
        return
    raise ValueError(dtype)
