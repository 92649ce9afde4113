"""The allocation-free decode attention (gr_paged_decode_attn_noalloc) against the
workspace entry point (gr_paged_decode_attn): the same kernels on the same inputs, so
the outputs must be identical.

Two calls in a row share the library's per-device scratch: the Llama-3-8B step shape
(B = 8, contexts uniform 256..4096, f16 KV, rows of up to 16 workgroups whose partial
states the last one merges), then a smaller one (the first three rows, half their
contexts), which finds the first call's partials and counters in the scratch.  Each
output is also held to the oracle's bar for f16 KV (relative L2 2e-3 overall and per
row).
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, rel_l2, row_rel_l2, say, torch_cuda

pytestmark = pytest.mark.gpu


def test_noalloc_attention_matches_workspace_call(orc):
    torch = torch_cuda()
    import continuous_quantized_decode_amd as gr
    gr.lib()
    wl = synth.WORKLOADS["llama3_8b"]
    ctx = synth.ctx_lens(wl)
    kv = synth.kv_state(wl, ctx, n_layers=1, extra_slot=False)
    pm = kv.pages
    q = synth.attn_query(np.random.default_rng(91), wl.batch, wl.n_q_heads, wl.head_dim)
    kp, vp = dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch)
    cases = [("full", np.arange(wl.batch), ctx),
             ("smaller", np.arange(3), np.maximum(ctx[:3] // 2, 1).astype(ctx.dtype))]
    for name, rows, c in cases:
        say(f"no-alloc attention, {name} call: B={len(rows)}, ctx {c.tolist()}")
        meta = gr.attn_meta(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.kv_dtype, pm.num_pages, pm.max_blocks,
                            int(c.max()))
        shape = gr.gr_attn_launch_shape(wl.kv_dtype, len(rows), wl.n_kv_heads, int(c.max()))
        assert shape["wg_per_row"] > 1  # partial states and arrival counters live in the scratch
        qd, bt, cd = dev(q[rows], torch), dev(pm.block_table[rows], torch), dev(c, torch)
        got = host(gr.gr_paged_decode_attn_noalloc(qd, kp, vp, bt, cd, meta))
        want_ws = host(gr.gr_paged_decode_attn(qd, kp, vp, bt, cd, meta))
        assert np.isfinite(got).all()
        assert np.array_equal(got, want_ws)
        want = orc.paged_attention(q[rows], kv.k_pools[0], kv.v_pools[0], wl.kv_dtype, pm.block_table[rows], c,
                                   wl.n_kv_heads)
        err, rerr = rel_l2(got, want), row_rel_l2(got, want)
        say(f"  identical to the workspace call; rel_l2 vs oracle {err:.3e}, worst row {rerr:.3e}")
        assert err <= 2e-3 and rerr <= 2e-3
