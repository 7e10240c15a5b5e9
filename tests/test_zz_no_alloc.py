"""The allocation-free attention call against the workspace call (needs an MI355X).

isb_sparse_pa_decode_noalloc keeps the split partials in the library's own
device array; its output must equal isb_sparse_pa_decode's bit for bit (the
same kernels), and both must match the oracle, on two calls in a row, the
second with a smaller input (the array keeps the first call's state).
"""
import numpy as np
import pytest
import torch

import indexer_selected_block_amd as isb
from indexer_selected_block_amd import workload as wl

from _util import attended_vmax, attn_tol, host_inputs, oracle_attention

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    isb.load_library()


def _case(base, reqs, ctx_lo, ctx_hi, top_k):
    cfg = wl.shrink(wl.CONFIGS[base], num_reqs=reqs, ctx_lo=ctx_lo, ctx_hi=ctx_hi, top_k=top_k,
                    pool_blocks=reqs * (-(-ctx_hi // 128)) + 64)
    w = wl.make_workload(cfg, device="cuda")
    layer = isb.DecodeLayer(w)
    layer.run()
    torch.cuda.synchronize()
    return cfg, w, layer


def _both(cfg, w, layer):
    args = (w.q, cfg.q_dtype, w.k_pool, w.v_pool, cfg.kv_dtype, w.k_scale, w.v_scale, layer.sparse_bt,
            layer.sparse_ctx, cfg.num_q_heads, cfg.num_kv_heads, w.sm_scale)
    ref = isb.sparse_pa_decode(*args, decode_query_len=cfg.query_len)
    out = torch.full_like(ref, float("nan"))
    isb.sparse_pa_decode_noalloc(*args, out, decode_query_len=cfg.query_len)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("base,big,small", [
    # 128 one-token rows of 16 blocks (two splits of eight waves), then 5 rows (four splits)
    ("fp8_decode", (128, 1500, 4000, 16), (5, 700, 5000, 16)),
    # MXFP4 pages, one page a wave: 40 rows of 16 blocks, then 3 rows of 10
    ("mxfp4", (40, 1800, 2100, 16), (3, 900, 1300, 10)),
])
def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row(base, big, small):
    for step, (reqs, lo, hi, k) in enumerate((big, small)):
        print(f"[no-alloc] {base} call {step}: {reqs} requests, top-k {k}", flush=True)
        cfg, w, layer = _case(base, reqs, lo, hi, k)
        need = isb.sparse_pa_workspace_bytes(cfg.num_tokens, cfg.num_q_heads, cfg.num_kv_heads,
                                             layer.sparse_bt.shape[1], cfg.kv_dtype)
        assert 0 < need <= 8 << 20, "the case must use the split partials"
        ref, out = _both(cfg, w, layer)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "differs from the workspace call"
        hi_ = host_inputs(w)
        sbt, sctx = layer.sparse_bt.cpu().numpy(), layer.sparse_ctx.cpu().numpy()
        o_ref = oracle_attention(hi_, sbt, sctx)
        err = np.abs(out.float().cpu().numpy() - o_ref).max()
        assert err <= attn_tol(cfg.kv_dtype, attended_vmax(hi_, sbt, sctx)), f"max |err| {err:.4g}"
