"""Standalone decode attention (gr_paged_decode_attn) at the workloads' real shapes.

The layer tests of the Llama-3-shaped workloads see almost nothing of the cached pages:
with random Q4_K weights the new token's own score dominates the softmax.  Here q is
drawn N(0, 1) (scores of standard deviation about 1 after 1/sqrt(D)), so every cached
token carries weight, over the real batch sizes, context-length distributions, page
pools and KV formats:

* Llama-3-8B step: B = 8, contexts uniform 256..4096, f16 KV, pages in random order;
* Qwen3-8B step: B = 32, contexts log-uniform 512..8192, q8_0 KV, a fragmented pool
  filled to 90 %;
* long-context stress: B = 64, contexts uniform 4096..32768, q8_0 KV scattered over a
  pool of about 1.3 M tokens: rows of several workgroups, each walking several groups of
  pages; the oracle checks a sample of rows (the four longest among them).

Bars: relative L2 2e-3 (f16) and 5e-3 (q8_0) against the fp64 oracle, over the whole
output and for every row on its own (the oracle reads the same stored K/V, so the
kernel-level difference is far below these; the layer-level bars are stated anyway).
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, rel_l2, row_rel_l2, say, torch_cuda

pytestmark = pytest.mark.gpu


def tol(kv_dtype):
    return 5e-3 if kv_dtype == synth.KV_Q8_0 else 2e-3


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


@pytest.fixture(scope="module")
def gr():
    import continuous_quantized_decode_amd as gr
    gr.lib()
    return gr


@pytest.mark.parametrize("name,sample", [("llama3_8b", None), ("qwen3_8b", None), ("longctx", 16)])
def test_attention_at_workload_shape(torch, gr, orc, name, sample):
    wl = synth.WORKLOADS[name]
    ctx = synth.ctx_lens(wl)
    say(f"attention {name}: B={wl.batch}, ctx {int(ctx.min())}..{int(ctx.max())}, kv {wl.kv_dtype}, "
        f"pool {wl.pool_kind}")
    kv = synth.kv_state(wl, ctx, n_layers=1, extra_slot=False)
    pm = kv.pages
    q = synth.attn_query(np.random.default_rng(77), wl.batch, wl.n_q_heads, wl.head_dim)
    shape = gr.gr_attn_launch_shape(wl.kv_dtype, wl.batch, wl.n_kv_heads, int(ctx.max()))
    say(f"  launch {shape}")
    if name == "longctx":
        assert shape["wg_per_row"] > 1  # rows of several workgroups whose states the last one merges
    meta = gr.attn_meta(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.kv_dtype, pm.num_pages, pm.max_blocks,
                        int(ctx.max()))
    got = host(gr.gr_paged_decode_attn(dev(q, torch), dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch),
                                       dev(pm.block_table, torch), dev(ctx, torch), meta))
    assert np.isfinite(got).all()
    rows = np.arange(wl.batch)
    if sample:
        longest = np.argsort(ctx)[-4:]
        rest = np.setdiff1d(rows, longest)
        rows = np.sort(np.concatenate([longest, np.random.default_rng(5).choice(rest, sample - 4, replace=False)]))
    say(f"  oracle over rows {rows.tolist()}")
    want = orc.paged_attention(q[rows], kv.k_pools[0], kv.v_pools[0], wl.kv_dtype, pm.block_table[rows], ctx[rows],
                               wl.n_kv_heads)
    err, rerr = rel_l2(got[rows], want), row_rel_l2(got[rows], want)
    say(f"  rel_l2 {err:.3e}, worst row {rerr:.3e}")
    assert err <= tol(wl.kv_dtype) and rerr <= tol(wl.kv_dtype)
    # the call is repeatable: the arrival counters were left at zero
    again = host(gr.gr_paged_decode_attn(dev(q, torch), dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch),
                                         dev(pm.block_table, torch), dev(ctx, torch), meta))
    assert np.array_equal(again, got)


def test_attention_workgroup_boundaries(torch, gr, orc):
    """Context lengths on either side of the workgroup and wave page ranges (16 pages
    per workgroup, 4 per wave at f16): rows whose last workgroup holds one page, or one
    token, next to rows of exactly one workgroup."""
    wl = synth.WORKLOADS["llama3_8b"]
    import dataclasses
    wl = dataclasses.replace(wl, batch=10, pool_kind="fill90")
    ctx = np.array([1, 16, 17, 64, 65, 255, 256, 257, 16 * 16 * 5, 16 * 16 * 5 + 1], np.int32)
    kv = synth.kv_state(wl, ctx, n_layers=1, extra_slot=False)
    pm = kv.pages
    q = synth.attn_query(np.random.default_rng(78), wl.batch, wl.n_q_heads, wl.head_dim)
    meta = gr.attn_meta(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.kv_dtype, pm.num_pages, pm.max_blocks,
                        int(ctx.max()))
    got = host(gr.gr_paged_decode_attn(dev(q, torch), dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch),
                                       dev(pm.block_table, torch), dev(ctx, torch), meta))
    want = orc.paged_attention(q, kv.k_pools[0], kv.v_pools[0], wl.kv_dtype, pm.block_table, ctx, wl.n_kv_heads)
    err = row_rel_l2(got, want)
    say(f"  worst row rel_l2 {err:.3e}")
    assert err <= 1e-4


def test_attention_many_workgroup_merge(torch, gr, orc):
    """Few rows with one long context: the work list gives the long row's (row, KV head)
    dozens of workgroups (the step's pages spread over the resident slots), so the last
    one merges their states over several rounds of loads; q8_0 and f16 pools, rows of
    1 and 2 tokens beside it."""
    import dataclasses
    for kv_dtype in (synth.KV_Q8_0, synth.KV_F16):
        wl = dataclasses.replace(synth.WORKLOADS["longctx"], batch=3, kv_dtype=kv_dtype, pool_kind="fill90")
        ctx = np.array([30001, 1, 2], np.int32)
        kv = synth.kv_state(wl, ctx, n_layers=1, extra_slot=False)
        pm = kv.pages
        q = synth.attn_query(np.random.default_rng(79), wl.batch, wl.n_q_heads, wl.head_dim)
        meta = gr.attn_meta(wl.n_q_heads, wl.n_kv_heads, wl.head_dim, kv_dtype, pm.num_pages, pm.max_blocks,
                            int(ctx.max()))
        got = host(gr.gr_paged_decode_attn(dev(q, torch), dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch),
                                           dev(pm.block_table, torch), dev(ctx, torch), meta))
        want = orc.paged_attention(q, kv.k_pools[0], kv.v_pools[0], kv_dtype, pm.block_table, ctx, wl.n_kv_heads)
        err = row_rel_l2(got, want)
        say(f"  kv {kv_dtype}: worst row rel_l2 {err:.3e}")
        assert err <= 1e-4
