"""GPU parity of the candidate merge (the merge step of context parallelism):
bit-exact against the oracle's merge and against the whole-row selection."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import indexer_selected_block_amd as isb
from oracle import decode as od

from _util import shard_candidates

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    isb.load_library()


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_oracle_shard_picks_is_bit_exact(seed):
    rng = np.random.default_rng(100 + seed)
    H, T, MB = 2, 7, int(rng.integers(2, 400))
    K = int(rng.integers(1, 33))
    if seed % 2:
        scores = rng.choice([-1.0, -0.0, 0.0, 0.5, np.nan, np.inf, -np.inf], size=(H, T, MB)).astype(np.float32)
    else:
        scores = np.round(rng.standard_normal((H, T, MB)), 1).astype(np.float32)
    lens = rng.integers(0, MB * 128 + 1, T).astype(np.int32)
    lens[0], lens[1] = 0, MB * 128
    G = int(rng.integers(1, 9))
    sc, ids = shard_candidates(scores, lens, G, K, rng)
    _say(f"merge seed {seed}: MB {MB} K {K} G {G} C {ids.shape[2]}")
    got = isb.topk_merge(torch.from_numpy(sc).cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(lens).cuda(),
                         1, K, MB)
    torch.cuda.synchronize()
    want = od.merge_candidates(sc, ids, lens, 1, K, MB)
    assert np.array_equal(got.cpu().numpy(), want)
    assert np.array_equal(want, od.topk_select(scores, lens, 1, K))


def test_context_parallel_rehearsal_at_long_context_shape():
    # 16 rows of 8192 blocks (1M-token contexts, ragged ends), top-k 32, the
    # blocks in 8 equal shards: every shard selected on the GPU as if it held
    # the whole row, the picks gathered with their scores, then merged.
    rng = np.random.default_rng(7)
    T, MB, K, G = 16, 8192, 32, 8
    scores = torch.from_numpy(rng.standard_t(3, size=(1, T, MB)).astype(np.float32))
    scores[0, 3, 100:140] = 2.5                                   # a run of ties
    lens = np.full(T, MB * 128, np.int32)
    lens[1::3] -= rng.integers(1, 128 * 900, len(lens[1::3])).astype(np.int32)
    dev = scores.cuda()
    span = MB // G
    picks, picked_scores = [], []
    for s in range(G):
        a, b = s * span, (s + 1) * span
        local_len = np.clip(lens.astype(np.int64) - a * 128, 0, (b - a) * 128).astype(np.int32)
        sel = isb.topk_select(dev[:, :, a:b].contiguous(), torch.from_numpy(local_len).cuda(), 1, K)
        ids = torch.where(sel >= 0, sel + a, sel)
        picks.append(ids)
        picked_scores.append(torch.where(sel >= 0, torch.gather(dev, 2, ids.clamp(min=0).long()), 0.0))
    cand_ids = torch.cat(picks, dim=2).contiguous()
    cand_sc = torch.cat(picked_scores, dim=2).contiguous()
    _say(f"cp rehearsal: {T} rows x {MB} blocks, {G} shards, {cand_ids.shape[2]} candidates a row")
    lens_d = torch.from_numpy(lens).cuda()
    got = isb.topk_merge(cand_sc, cand_ids, lens_d, 1, K, MB)
    whole = isb.topk_select(dev, lens_d, 1, K)
    again = [isb.topk_merge(cand_sc, cand_ids, lens_d, 1, K, MB) for _ in range(8)]   # repeated calls agree
    torch.cuda.synchronize()
    assert all(torch.equal(x, got) for x in again)
    want = od.topk_select(scores.numpy(), lens, 1, K)
    assert np.array_equal(whole.cpu().numpy(), want)
    assert np.array_equal(got.cpu().numpy(), want)
