#!/usr/bin/env python3
"""Benchmark of one indexed block-sparse paged-attention decode layer on one MI355X.

A step is one pass of the whole path over one batch: index_score, then
select_attend (top-k selection, the sparse page table and the split-K
attention with its merge, in one launch where the shapes allow), on
the fp8 decode workload (128 requests x 1 token, contexts U{16384..65536},
fp8 K/V and index cache, 16 query heads per KV head, top-k 16 blocks) unless
--config names another.  Inputs are synthetic and resident in HBM before the
timed region starts.

Each step uses the next of --layers independent copies of the inputs, so the
pages a step reads were not read by the step before it.

Prints one JSON line: decode tokens/s of the whole step (value), the
attended-KV HBM rate of the attention, per-call durations (the step's two
calls, and the path's separate calls index_score, topk_select_emit and
sparse_pa_decode) taken as differences between back-to-back passes of K steps
timed with HIP events on the launch stream (with a 512 MB scrub between the
steps of every pass, so no step finds its inputs in the last-level cache), a
roofline entry for the dominant kernel (and one for the attention alone), the
measured ceilings of the two large launches (their page reads with no
arithmetic, in their own grids), a device copy's measured rate at the
attention's transfer size and at 1 GiB next to the nominal peak, and the CPU
oracle timed on a bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode tokens/s + attended-KV HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
IDX_BYTES = {"bf16": 256, "fp8": 128, "mxfp4": 68}           # bytes per index key
KV_BYTES = {"bf16": 256, "fp8": 128, "mxfp4": 68}            # bytes per token, one of K or V
Q_BYTES = {"bf16": 2, "e4m3": 1}
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="fp8_decode")
    ap.add_argument("--layers", type=int, default=8,
                    help="independent copies of the layer's inputs, used round-robin, so a "
                         "step does not find the pages it reads in the 256 MB last-level "
                         "cache (a step's pages were last read 8 steps, over 500 MB of "
                         "attended pages and 5 GB of index keys, earlier)")
    ap.add_argument("--scrub-mb", type=int, default=512,
                    help="MB a copy moves between the steps of the per-call timing passes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU oracle baseline (0 skips it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 10 times (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 10}))


def measured_copy(nbytes_moved):
    """Device copy (torch's copy kernel) moving `nbytes_moved` bytes (half read,
    half written) per launch, cycling over enough buffer pairs to exceed the
    256 MB last-level cache; GB/s of the average launch, HIP events."""
    import torch
    half = max(1 << 20, nbytes_moved // 2)
    pairs = max(2, -(-(600 << 20) // (2 * half)))
    bufs = [(torch.ones(half, dtype=torch.uint8, device="cuda"),
             torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(pairs)]
    reps = max(2 * pairs, 20)
    for i in range(pairs):
        bufs[i][1].copy_(bufs[i][0])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        src, dst = bufs[i % pairs]
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    del bufs
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * half, "avg_us": round(us, 2), "GBps": round(2 * half / (us * 1e-6) / 1e9, 1)}


def token_geometry(L):
    """Per query token of a layer's batch: (request, causal length).  Decode
    batches: token r q + i of request r, L_t = max(0, L_r - (q - 1 - i));
    ragged prefill batches: each token's own request id and position + 1."""
    b = getattr(L, "b", None)
    if b is not None:
        return list(zip(b.query_req_id.cpu().tolist(), [p + 1 for p in b.query_abs_pos.cpu().tolist()]))
    ql = L.w.cfg.query_len
    return [(r, max(0, Lr - (ql - 1 - i))) for r, Lr in enumerate(L.w.seq_lens.cpu().tolist()) for i in range(ql)]


def distinct_attended_tokens(L, topk):
    """K/V positions the attention must read at least once: per request and KV
    head, the union over the request's query tokens of their selected blocks,
    each block up to the longest causal reach of a token that selects it (the
    tokens of one request can select the same blocks)."""
    geo = token_geometry(L)
    tk = topk.cpu().tolist()  # [H_kv][T][K]
    total = 0
    for g in range(L.w.cfg.num_kv_heads):
        reach = {}
        for t, (r, Lt) in enumerate(geo):
            for b in tk[g][t]:
                if b >= 0:
                    reach[(r, b)] = max(reach.get((r, b), 0), min(128, Lt - 128 * b))
        total += sum(reach.values())
    return total


def algorithmic_bytes(L, sparse_ctx, topk):
    """Bytes each kernel must move for this batch: the index keys of every
    request once (up to the farthest position one of its tokens sees), the
    queries, the table entries and token positions read, the scores,
    selection, page table and outputs written; for the attention the K and V
    bytes of the positions attended, each distinct position once (rows of one
    request that select the same block need its bytes once).  Split partials
    and re-reads are not counted."""
    cfg = L.w.cfg
    geo = token_geometry(L)
    T = len(geo)
    reach = {}
    for r, Lt in geo:
        reach[r] = max(reach.get(r, 0), Lt)
    n_req_blocks = sum(-(-x // 128) for x in reach.values())
    n_tok_blocks = sum(-(-Lt // 128) for _, Lt in geo)
    per_token_in = 8 * T if getattr(L, "b", None) is not None else 4 * len(reach)   # positions / lengths
    qidx = T * cfg.num_idx_heads * 128 * Q_BYTES[cfg.qidx_dtype]
    score = (sum(reach.values()) * IDX_BYTES[cfg.idx_dtype] + qidx + 4 * n_req_blocks + per_token_in
             + 4 * cfg.num_kv_heads * n_tok_blocks)
    rows = T * cfg.num_kv_heads
    slots = cfg.top_k * cfg.pages_per_block
    # top-k + emit: scores and lengths in, the table entries the selection names
    # in, the selection, the page table and the lengths out
    topk_emit = (4 * cfg.num_kv_heads * n_tok_blocks + per_token_in + 4 * rows * cfg.top_k
                 + 4 * rows * cfg.top_k + 4 * rows * (slots + 1))
    ctx = sparse_ctx.cpu().long()
    attended = distinct_attended_tokens(L, topk) * 2 * KV_BYTES[cfg.kv_dtype]
    ptok = 128 // cfg.pages_per_block
    pages = int(((ctx + ptok - 1) // ptok).sum())
    attn = (attended + T * cfg.num_q_heads * 128 * (Q_BYTES[cfg.q_dtype] + 2) + 4 * pages + 4 * rows)
    per_row = int(ctx.sum()) * 2 * KV_BYTES[cfg.kv_dtype]
    return {"index_score": score, "topk_select_emit": topk_emit, "sparse_pa_decode": attn}, attended, per_row


def index_flops(L):
    """Multiply-adds (x2) the scorer must do: each index query row against each
    of its token's causally valid keys, 128 dims."""
    return 2 * 128 * L.w.cfg.num_idx_heads * sum(Lt for _, Lt in token_geometry(L))


def scorer_is_wide(cfg, ragged=False):
    """More than 16 tokens or 64 index query rows a request, or a ragged
    prefill batch: the scorer that holds a block's keys in registers and runs
    them against 16-row query tiles on MFMA; its bound is the MFMA rate, not
    HBM."""
    return ragged or cfg.query_len > 16 or cfg.query_len * cfg.num_idx_heads > 64


# dense MFMA peaks of MI355X (TFLOP/s) for the scorer's operand types: bf16
# operands (bf16 / fp8 keys converted to bf16, or MXFP4 keys with a bf16 query),
# or fp8 / MXFP4 keys with an e4m3 query on the scaled fp8/fp4 instruction
# (fp8 rate)
def mfma_peak_tflops(cfg):
    return 5000.0 if (cfg.idx_dtype in ("fp8", "mxfp4") and cfg.qidx_dtype == "e4m3") else 2500.0


def kernel_sources_sha():
    """Hash of each kernel's source file, to tell whether stored counters still apply."""
    csrc = os.path.join(ROOT, "indexer_selected_block_amd", "csrc")
    files = {"index_score": "index_score.hip", "topk_select_emit": "topk_select.hip",
             "sparse_pa_decode": "sparse_pa.hip", "select_attend": "sparse_pa.hip"}
    common = b"".join(open(os.path.join(csrc, f), "rb").read()
                      for f in ("isb_device.h", "isb_host.h", "select_device.h", "grid_maps.h"))
    return {k: hashlib.sha256(common + open(os.path.join(csrc, f), "rb").read()).hexdigest()[:16]
            for k, f in files.items()}


def stored_traffic(config, kernel, sha):
    """HBM bytes per call from the committed rocprofv3 counter summaries
    (profiles/*.txt lines "traffic <config> <kernel> source_sha=.. bytes_per_launch=.."),
    if they were taken on this exact kernel source and workload; else None."""
    try:
        names = sorted(os.listdir(PROFILES))
    except OSError:
        return None
    for name in names:
        if not name.endswith(".txt"):
            continue
        with open(os.path.join(PROFILES, name)) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 5 and parts[0] == "traffic" and parts[1] == config and parts[2] == kernel:
                    fields = dict(x.split("=", 1) for x in parts[3:])
                    if fields.get("source_sha") == sha:
                        return int(fields["bytes_per_launch"])
    return None


def _oracle_worker(folder, fields, wid, nworkers, budget_s, barrier, results):
    """One CPU process of the oracle baseline: requests wid, wid + nworkers, ...
    of the saved sample, cycling, until its budget is spent; reports (query
    tokens, requests, seconds)."""
    import numpy as np

    from oracle import decode as od
    from oracle import formats

    d = {k: np.load(os.path.join(folder, k + ".npy"), mmap_mode="r")
         for k in ("idx", "k", "v", "off", "lens", "q", "q_idx")}
    ql, ppb = fields["query_len"], fields["ppb"]
    off, lens = np.array(d["off"]), np.array(d["lens"])
    live = [r for r in range(len(lens)) if lens[r] > 0]
    mine = live[wid::nworkers] or live[:1]
    barrier.wait(timeout=600)
    t0 = time.perf_counter()
    tokens = nreq = 0
    i = 0
    while True:
        r = mine[i % len(mine)]
        i += 1
        L, b0, b1 = int(lens[r]), int(off[r]), int(off[r + 1])
        nb = b1 - b0
        q = formats.decode_query(np.array(d["q"][r * ql:(r + 1) * ql]), fields["q_dtype"])
        q_idx = formats.decode_query(np.array(d["q_idx"][r * ql:(r + 1) * ql]), fields["qidx_dtype"])
        od.decode_layer(q, q_idx, d["idx"][b0:b1], fields["idx_dtype"], fields["idx_scale"],
                        d["k"][b0 * ppb:b1 * ppb], d["v"][b0 * ppb:b1 * ppb], fields["kv_dtype"],
                        fields["k_scale"], fields["v_scale"], np.arange(nb, dtype=np.int64)[None, :], [L], ql,
                        fields["num_kv_heads"], nb, fields["top_k"], ppb, fields["sm_scale"])
        tokens += ql
        nreq += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    results.put((tokens, nreq, time.perf_counter() - t0))


def cpu_baseline(w, budget_s, max_sample_bytes=3 << 30):
    """The oracle, as it is, on whole requests of the same workload, in
    parallel processes over this host's cores (one numpy / BLAS thread each),
    until each has spent the budget; tokens/s of all of them together.  The
    sample is the batch's requests in order, as many as fit in
    max_sample_bytes of host copies of their pages."""
    import multiprocessing as mp
    import tempfile

    import numpy as np

    cfg = w.cfg
    ppb = cfg.pages_per_block
    affinity = len(os.sched_getaffinity(0))
    # one process a core, at most 16: the CPU share of one GPU on the boxes
    # this runs on
    nproc = max(1, min(affinity, 16))
    lens_all = w.seq_lens.cpu().numpy()
    per_block = w.idx_pool.shape[1] + 2 * ppb * w.k_pool.shape[1]
    reqs, nbytes = [], 0
    for r, L in enumerate(lens_all):
        nb = -(-int(L) // 128)
        if reqs and nbytes + nb * per_block > max_sample_bytes:
            break
        reqs.append(r)
        nbytes += nb * per_block
    # each sampled request's pages copied to the host (not timed), renumbered
    lens = lens_all[reqs]
    nblk = [-(-int(L) // 128) for L in lens]
    off = np.concatenate([[0], np.cumsum(nblk)]).astype(np.int64)
    ids = torch_cat_blocks(w, reqs, nblk)
    kv = lambda p: p.view(p.shape[0] // ppb, -1)[ids].cpu().reshape(len(ids) * ppb, -1).numpy()  # noqa: E731
    ql = cfg.query_len
    toks = [r * ql + i for r in reqs for i in range(ql)]
    fields = dict(query_len=ql, ppb=ppb, q_dtype=cfg.q_dtype, qidx_dtype=cfg.qidx_dtype,
                  idx_dtype=cfg.idx_dtype, kv_dtype=cfg.kv_dtype, num_kv_heads=cfg.num_kv_heads, top_k=cfg.top_k,
                  idx_scale=w.idx_scale, k_scale=w.k_scale, v_scale=w.v_scale, sm_scale=w.sm_scale)
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    with tempfile.TemporaryDirectory() as tmp:
        for name, arr in (("idx", w.idx_pool[ids].cpu().numpy()), ("k", kv(w.k_pool)), ("v", kv(w.v_pool)),
                          ("off", off), ("lens", lens), ("q", w.q[toks].cpu().numpy()),
                          ("q_idx", w.q_idx[toks].cpu().numpy())):
            np.save(os.path.join(tmp, name + ".npy"), arr)
            del arr
        for k in env:
            os.environ[k] = "1"
        try:
            ctx = mp.get_context("spawn")    # fresh interpreters: no GPU state is inherited
            barrier, results = ctx.Barrier(nproc), ctx.Queue()
            procs = [ctx.Process(target=_oracle_worker, args=(tmp, fields, i, nproc, budget_s, barrier, results))
                     for i in range(nproc)]
            for p in procs:
                p.start()
            got = []
            deadline = time.time() + budget_s + 900
            while len(got) < nproc:
                try:
                    got.append(results.get(timeout=5))
                except Exception:  # queue.Empty: check that every worker is still alive
                    dead = [p.exitcode for p in procs if p.exitcode not in (None, 0)]
                    if dead or time.time() > deadline:
                        for p in procs:
                            p.kill()
                        raise RuntimeError(f"CPU oracle workers failed (exit codes {dead})")
            for p in procs:
                p.join()
        finally:
            for k, v in env.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    tokens = sum(g[0] for g in got)
    nreq = sum(g[1] for g in got)
    rate = sum(g[0] / g[2] for g in got)    # the processes run side by side
    return {"value": rate, "unit": "tokens/s", "cores": nproc, "kind": "oracle",
            "sample": f"the first {len(reqs)} of {len(lens_all)} requests of the same workload, whole; "
                      f"{nproc} processes, one a core ({affinity} cores in this process's affinity), each "
                      f"cycling over its share for ~{budget_s:.0f} s: {nreq} requests ({tokens} query tokens) "
                      f"in all; numpy float64 with BLAS limited to 1 thread a process"}


def torch_cat_blocks(w, reqs, nblk):
    """Device block ids of the given requests' blocks, request after request."""
    import torch
    parts = [w.block_table[r, :n].long() for r, n in zip(reqs, nblk) if n]
    return torch.cat(parts) if parts else torch.zeros(0, dtype=torch.long, device=w.block_table.device)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the path has no "
                                   "multi-GPU part (rows are independent; each GPU would run "
                                   "it on its own requests)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import indexer_selected_block_amd as isb
    from indexer_selected_block_amd import workload as wl

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    ragged = args.config in wl.RAGGED_CHUNKS
    cfg = wl.ragged_config(args.config) if ragged else wl.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    print(f"[bench] building {args.config} x{args.layers} on {torch.cuda.get_device_name(0)}",
          file=sys.stderr, flush=True)
    layers = []
    for li in range(args.layers):
        c = cfg if li == 0 else dataclasses.replace(cfg, seed=cfg.seed + 1000 * li)
        w = wl.make_workload(c, device=dev)
        if ragged:  # a prefill batch: the requests' chunks, each token with its own request and position
            layers.append(isb.PrefillLayer(w, wl.ragged_batch(w, wl.RAGGED_CHUNKS[args.config], seed=li)))
        else:
            layers.append(isb.DecodeLayer(w))
    torch.cuda.synchronize()

    for s in range(args.warmup):
        layers[s % len(layers)].run()
    torch.cuda.synchronize()

    # ---- timed region: K whole steps, nothing else on the stream
    t0 = time.perf_counter()
    for s in range(args.steps):
        layers[s % len(layers)].run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # live query tokens: pad requests (length 0) compute nothing and are not counted
    T = (layers[0].b.num_tokens if ragged else int((layers[0].w.seq_lens > 0).sum()) * cfg.query_len)
    ms_per_step = 1000.0 * elapsed / args.steps

    # ---- per-kernel durations, each in its place in the step: passes of K
    # steps that stop after a given call, run back to back and timed with HIP
    # events on the launch stream; a call's duration is the difference between
    # the pass that ends with it and the pass that ends just before it (an
    # event between two kernels would add its own idle gap, these do not).
    stream = torch.cuda.current_stream(dev)

    def call_index(L):
        w, c = L.w, L.w.cfg
        if ragged:
            isb.index_score_prefill(L.b.q_idx, c.qidx_dtype, w.idx_pool, c.idx_dtype, w.idx_scale, w.block_table,
                                    L.b.query_req_id, L.b.query_abs_pos, c.num_kv_heads, c.max_blocks,
                                    scores=L.scores)
            return
        isb.index_score(w.q_idx, c.qidx_dtype, w.idx_pool, c.idx_dtype, w.idx_scale, w.block_table,
                        w.seq_lens, c.query_len, c.num_kv_heads, c.max_blocks, scores=L.scores)

    def call_topk(L):
        w, c = L.w, L.w.cfg
        if ragged:
            isb.topk_select_emit_prefill(L.scores, L.b.query_req_id, L.b.query_abs_pos, c.top_k, w.block_table,
                                         c.pages_per_block, topk_idx=L.topk, sparse_bt=L.sparse_bt,
                                         sparse_ctx=L.sparse_ctx)
            return
        isb.topk_select_emit(L.scores, w.seq_lens, c.query_len, c.top_k, w.block_table, c.pages_per_block,
                             topk_idx=L.topk, sparse_bt=L.sparse_bt, sparse_ctx=L.sparse_ctx)

    def call_attend(L):
        w, c = L.w, L.w.cfg
        if ragged:
            isb.sparse_pa_prefill(L.b.q, c.q_dtype, w.k_pool, w.v_pool, c.kv_dtype, w.k_scale, w.v_scale,
                                  L.sparse_bt, L.sparse_ctx, c.num_q_heads, c.num_kv_heads, w.sm_scale,
                                  out=L.out, workspace=L.workspace)
            return
        isb.sparse_pa_decode(w.q, c.q_dtype, w.k_pool, w.v_pool, c.kv_dtype, w.k_scale, w.v_scale,
                             L.sparse_bt, L.sparse_ctx, c.num_q_heads, c.num_kv_heads, w.sm_scale,
                             out=L.out, workspace=L.workspace, decode_query_len=c.query_len)

    def call_select_attend(L):
        w, c = L.w, L.w.cfg
        if ragged:
            isb.select_attend_prefill(L.scores, L.b.query_req_id, L.b.query_abs_pos, c.top_k, w.block_table, L.b.q,
                                      c.q_dtype, w.k_pool, w.v_pool, c.kv_dtype, w.k_scale, w.v_scale,
                                      c.num_q_heads, w.sm_scale, topk_idx=L.topk, sparse_bt=L.sparse_bt,
                                      sparse_ctx=L.sparse_ctx, out=L.out, workspace=L.workspace)
            return
        isb.select_attend(L.scores, w.seq_lens, c.query_len, c.top_k, w.block_table, w.q, c.q_dtype, w.k_pool,
                          w.v_pool, c.kv_dtype, w.k_scale, w.v_scale, c.num_q_heads, w.sm_scale, topk_idx=L.topk,
                          sparse_bt=L.sparse_bt, sparse_ctx=L.sparse_ctx, out=L.out, workspace=L.workspace)

    def pass_ms(calls):
        """Average ms of one step made of `calls`, over K steps (HIP events)."""
        for s in range(min(args.warmup, 4)):
            for f in calls:
                f(layers[s % len(layers)])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.steps):
            for f in calls:
                f(layers[s % len(layers)])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # A scrub between steps of these passes (a copy that moves --scrub-mb MB
    # through the memory system, in every pass alike, so that it cancels in
    # the differences) leaves nothing of a step's inputs in the 256 MB
    # last-level cache for the next step, whatever the workload's size.
    scrub_half = max(1, args.scrub_mb // 2) << 20
    scrub_src = torch.ones(scrub_half, dtype=torch.uint8, device=dev)
    scrub_dst = torch.empty_like(scrub_src)

    def scrub(L):
        scrub_dst.copy_(scrub_src)

    # the passes in turn, three times; each pass's median, so that one noisy
    # pass does not move a difference
    reps = {"s": [], "i": [], "it": [], "ita": [], "step": []}
    for _ in range(3):
        reps["s"].append(pass_ms([scrub]))
        reps["i"].append(pass_ms([call_index, scrub]))
        reps["it"].append(pass_ms([call_index, call_topk, scrub]))
        reps["ita"].append(pass_ms([call_index, call_topk, call_attend, scrub]))
        reps["step"].append(pass_ms([call_index, call_select_attend, scrub]))
    t_s, t_i, t_it, t_ita, t_step = (sorted(reps[k])[1] for k in ("s", "i", "it", "ita", "step"))
    dur_ms = {"index_score": t_i - t_s, "topk_select_emit": t_it - t_i, "sparse_pa_decode": t_ita - t_it,
              "select_attend": t_step - t_i}
    ceilings = time_ceilings(layers, pass_ms, scrub, t_s, stream, ragged)
    # the same with one input copy: the attention's pages can stay in the
    # last-level cache from the step before (reported apart, never as value)
    all_layers = layers
    layers = layers[:1]
    warm = [pass_ms([call_index, call_topk, call_attend]) - pass_ms([call_index, call_topk]) for _ in range(3)]
    warm_attend = sorted(warm)[1]
    layers = all_layers
    names = ["index_score", "topk_select_emit", "sparse_pa_decode"]

    w0 = layers[0].w
    # the copies differ in lengths and selections: bytes are averaged over the
    # copies the timed steps cycle through, like the durations
    per_copy = [algorithmic_bytes(L, L.sparse_ctx, L.topk) for L in layers]
    alg = {k: sum(a[k] for a, _, _ in per_copy) / len(per_copy) for k in per_copy[0][0]}
    attended = sum(x for _, x, _ in per_copy) / len(per_copy)
    attended_rows = sum(x for _, _, x in per_copy) / len(per_copy)
    shas = kernel_sources_sha()

    flops = sum(index_flops(L) for L in layers) / len(layers)

    def roof(kernel):
        if kernel == "index_score" and scorer_is_wide(cfg, ragged):
            tflops = flops / (dur_ms[kernel] * 1e-3) / 1e12
            peak = mfma_peak_tflops(cfg)
            return {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4),
                    "traffic": stored_traffic(args.config, kernel, shas[kernel]),
                    "kernel": kernel, "avg_ms": round(dur_ms[kernel], 5),
                    "algorithmic_flops": int(round(flops)), "algorithmic_bytes": int(round(alg[kernel]))}
        gbps = alg[kernel] / (dur_ms[kernel] * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "traffic": stored_traffic(args.config, kernel, shas[kernel]),
                "kernel": kernel, "avg_ms": round(dur_ms[kernel], 5),
                "algorithmic_bytes": int(round(alg[kernel]))}

    dominant = max(names, key=lambda n: dur_ms[n])  # among the separate calls
    attn_gbps = attended / (dur_ms["sparse_pa_decode"] * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e4m3 K->bf16 and V->f16 mfma, f32 accumulate" if cfg.kv_dtype == "fp8"
                  else f"{cfg.kv_dtype} in, f32 accumulate"),
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "requests": cfg.total_reqs,
                   "query_len": "ragged" if ragged else cfg.query_len, "tokens_per_step": T,
                   "token_rows": T if ragged else cfg.num_tokens,
                   "top_k": cfg.top_k,
                   "q_heads_per_kv": cfg.num_q_heads // cfg.num_kv_heads,
                   "index_heads": cfg.num_idx_heads, "kv_cache": cfg.kv_dtype,
                   "index_cache": cfg.idx_dtype, "layers": args.layers},
        "attended_kv_GBps": round(attn_gbps, 1),
        "attended_kv_pct_hbm_peak": round(100 * attn_gbps / HBM_PEAK_GBPS, 2),
        "attended_kv_bytes": {"distinct": int(round(attended)), "summed_over_rows": int(round(attended_rows))},
        "step_launches": (["index_score_prefill", "select_attend_prefill"] if ragged
                          else ["index_score", "select_attend"]),
        "kernel_ms": {k: round(v, 5) for k, v in dur_ms.items()},
        "kernel_ms_method": "differences of back-to-back passes of K steps ending after each call (HIP events; median of 3 rounds)",
        "sparse_pa_decode_ms_one_input_copy": round(warm_attend, 5),
        "roofline": roof(dominant),
        "roofline_sparse_pa_decode": roof("sparse_pa_decode"),
    }
    if dominant != "index_score":
        result["roofline_index_score"] = roof("index_score")
    for k, c in ceilings.items():
        kernel = {"index_gather": "index_score", "attention_gather": "sparse_pa_decode"}[k]
        gbps = alg[kernel] / (c["avg_ms"] * 1e-3) / 1e9
        c.update({"GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                  "kernel_over_ceiling": round(dur_ms[kernel] / c["avg_ms"], 3),
                  "bytes": int(round(alg[kernel]))})
    result["ceilings"] = ceilings
    result["measured_copy"] = {"at_attention_size": measured_copy(int(alg["sparse_pa_decode"])),
                               "at_1GiB": measured_copy(1 << 30)}
    if args.cpu_seconds > 0 and not ragged:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w0, args.cpu_seconds)
    else:  # the oracle baseline is taken on decode batches
        result["cpu_baseline"] = None
    result["write_cache"] = None if ragged else time_writer(isb, w0, stream, args.steps)
    print(json.dumps(result))


def time_ceilings(layers, pass_ms, scrub, t_scrub, stream, ragged=False):
    """The measurement kernels of libisb_ceiling on the same inputs and
    passes as the layer's calls: the index scan's and the attention's page
    reads with no arithmetic, in their grids.  Per launch, as the passes'
    difference to the scrub alone."""
    import ctypes

    import torch

    from indexer_selected_block_amd import binding as bd
    from indexer_selected_block_amd.build import CEILING_LIB_PATH

    lib = ctypes.CDLL(CEILING_LIB_PATH)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.isb_ceiling_index_gather.argtypes = [P, P, I, I64, P, I, P, I, I, I, I, P]
    lib.isb_ceiling_attention_gather.argtypes = [P, P, P, I, I64, P, I, P, I, I, I, P, ctypes.c_size_t]
    lib.isb_ceiling_attention_words.argtypes = [I, I, I, I]
    lib.isb_ceiling_attention_words.restype = ctypes.c_size_t
    cfg = layers[0].w.cfg
    st = ctypes.c_void_p(stream.cuda_stream)
    dev = layers[0].w.q.device
    idx_out = torch.empty((cfg.total_reqs, cfg.max_blocks), dtype=torch.float32, device=dev)
    T = layers[0].sparse_ctx.shape[0] // cfg.num_kv_heads
    words = lib.isb_ceiling_attention_words(T, cfg.num_kv_heads, layers[0].sparse_bt.shape[1],
                                            bd._code(cfg.kv_dtype))
    att_out = torch.empty((max(int(words), 1),), dtype=torch.int32, device=dev)

    def index_gather(L):
        w = L.w
        rc = lib.isb_ceiling_index_gather(st, w.idx_pool.data_ptr(), bd._code(cfg.idx_dtype), w.idx_pool.shape[0],
                                          w.block_table.data_ptr(), w.block_table.shape[1], w.seq_lens.data_ptr(),
                                          w.seq_lens.shape[0], cfg.query_len, cfg.num_idx_heads, cfg.max_blocks,
                                          idx_out.data_ptr())
        if rc:
            raise RuntimeError(f"isb_ceiling_index_gather: status {rc}")

    def attention_gather(L):
        w = L.w
        # a prefill batch's rows share pages: read through the caches, as a
        # decode_query_len above 1 asks for
        rc = lib.isb_ceiling_attention_gather(st, w.k_pool.data_ptr(), w.v_pool.data_ptr(), bd._code(cfg.kv_dtype),
                                              w.k_pool.shape[0], L.sparse_bt.data_ptr(), L.sparse_bt.shape[1],
                                              L.sparse_ctx.data_ptr(), T, T if ragged else cfg.query_len,
                                              cfg.num_kv_heads, att_out.data_ptr(), att_out.numel())
        if rc:
            raise RuntimeError(f"isb_ceiling_attention_gather: status {rc}")

    out = {}
    kinds = [("attention_gather", attention_gather)]
    if not scorer_is_wide(cfg, ragged):
        kinds.insert(0, ("index_gather", index_gather))
    for name, f in kinds:
        t = sorted(pass_ms([f, scrub]) for _ in range(3))[1] - t_scrub
        out[name] = {"avg_ms": round(t, 5)}
    out["index_gather" if "index_gather" in out else "attention_gather"]["method"] = (
        "the same page reads, grid and cache policy as the call, no arithmetic (libisb_ceiling); "
        "per launch over the input copies, with the scrub between steps, like the calls")
    return out


def writer_bytes(cfg, live_tokens):
    """Algorithmic bytes of one isb_write_cache launch: the bf16 inputs of the
    live tokens read once, their stored bytes written once (fp8 1 B, bf16 2 B
    an element, MXFP4 64 B of codes and 4 scale bytes a 128-dim vector)."""
    stored = {"fp8": 128, "bf16": 256, "mxfp4": 68}
    vecs_kv = 2 * cfg.num_kv_heads
    read = live_tokens * (vecs_kv + 1) * 256
    write = live_tokens * (vecs_kv * stored[cfg.kv_dtype] + stored[cfg.idx_dtype])
    return read + write


def time_writer(isb, w, stream, steps):
    """The cache write in front of a step: the step's new tokens (one per
    query row, pad rows included in the launch) written into the workload's
    pools, K launches back to back, HIP events on the launch stream.  Runs
    last: it overwrites the last tokens of every request."""
    import torch
    cfg = w.cfg
    g = torch.Generator(device=w.k_pool.device).manual_seed(cfg.seed + 77)
    T, H = cfg.num_tokens, cfg.num_kv_heads
    k_new, v_new = (torch.randn((T, H, 128), generator=g, device=w.k_pool.device).to(torch.bfloat16)
                    for _ in range(2))
    i_new = torch.randn((T, 128), generator=g, device=w.k_pool.device).to(torch.bfloat16)

    # arguments checked once, then bare launches: the kernel, not the
    # binding's per-call checks, sets the rate
    call = isb.write_cache_launcher(k_new, v_new, i_new, w.block_table, w.seq_lens, cfg.query_len, w.k_pool,
                                    w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, w.idx_pool, cfg.idx_dtype,
                                    w.idx_scale)

    # the same write with the fused QK-norm and a NeoX rope over 64 dims on K
    # and the index keys (unit norm weights, tables up to the longest request)
    rot = 64
    npos = int(w.seq_lens.max().item())
    ang = torch.arange(npos, device=w.k_pool.device, dtype=torch.float64)[:, None] * \
        (10000.0 ** (-torch.arange(0, rot, 2, device=w.k_pool.device, dtype=torch.float64) / rot))[None, :]
    cos, sin = torch.cos(ang).float().contiguous(), torch.sin(ang).float().contiguous()
    ones = torch.ones(128, device=w.k_pool.device, dtype=torch.float32)
    nr = isb.norm_rope(ones, 1e-6, cos, sin, rot, True)
    call_nr = isb.write_cache_launcher(k_new, v_new, i_new, w.block_table, w.seq_lens, cfg.query_len, w.k_pool,
                                       w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, w.idx_pool, cfg.idx_dtype,
                                       w.idx_scale, nr, nr)

    def timed(f):
        for _ in range(4):
            f()
        reps = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / steps)
        return sorted(reps)[1]

    ms, ms_nr = timed(call), timed(call_nr)
    live = int((w.seq_lens > 0).sum()) * cfg.query_len
    nbytes = writer_bytes(cfg, live)
    return {"kernel": "write_cache", "avg_ms": round(ms, 5), "tokens": live, "algorithmic_bytes": nbytes,
            "achieved_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "avg_ms_with_norm_rope": round(ms_nr, 5),
            "note": "cache write in front of the step, outside value; back-to-back calls timed with HIP "
                    "events, median of 3 (at a decode step's size the host's call rate, ~4-5 us a call, "
                    "bounds this; the kernel trace gives the kernel alone); with_norm_rope: QK-norm and a "
                    "64-dim NeoX rope on K and the index keys"}


if __name__ == "__main__":
    main()
