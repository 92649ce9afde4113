"""GPU parity of whole decode layers and stacks against the fp64 oracle (C ABI).

Bars (relative L2 over each layer's [B, hidden] output, the GPU running the stack
end to end): 2e-3 for f32 / f16 KV, 5e-3 for q8_0 KV.
"""
import dataclasses

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


def upload_layer(gr, torch, lw):
    t = {k: dev(getattr(lw, k), torch) for k in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up",
                                                  "w_down")}
    if lw.q_norm is not None:
        t["q_norm"] = dev(lw.q_norm, torch)
        t["k_norm"] = dev(lw.k_norm, torch)
    for k in ("tq", "tk", "tv", "to", "tgate", "tup", "tdown"):
        t[k] = getattr(lw, k)
    return t, gr.layer_weights(t)


def cfg_of(gr, wl):
    return gr.layer_cfg(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.ffn, wl.rms_eps, wl.rope_theta,
                        wl.rope_style, wl.qk_norm, wl.kv_dtype)


def tiny(**rep):
    return dataclasses.replace(synth.WORKLOADS["tiny"], **rep)


LAYER_CASES = [
    dict(ctx=[128]),                                                    # the tiny workload as stated
    dict(ctx=[0, 15, 16, 17, 128], batch=5),
    dict(ctx=[5, 64, 200], batch=3, qk_norm=True),
    dict(ctx=[31, 32, 47], batch=3, kv_dtype=synth.KV_F16, rope_style=synth.ROPE_NORM),
    dict(ctx=[100, 1, 63], batch=3, kv_dtype=synth.KV_Q8_0, qk_norm=True),
    dict(ctx=[10] * 9, batch=9, kv_dtype=synth.KV_F16),                # two batch tiles
    dict(ctx=[300, 2, 77, 150, 19, 64, 33, 5, 1, 0, 250, 99], batch=12, kv_dtype=synth.KV_Q8_0, w_down=synth.W_Q6_K,
         head_dim=128, n_q_heads=2, n_kv_heads=2),
    # FFN wide enough for the tile-loop gate/up GEMM (528 gate/up tile pairs)
    dict(ctx=[40, 7, 300], batch=3, ffn=8448),
    dict(ctx=[20, 90], batch=2, ffn=8448, w_other=synth.W_Q6_K, kv_dtype=synth.KV_F16),
    # Q5_K / Q8_0 weight rows in the fused GEMMs (QKV, O, gate/up + SwiGLU, down)
    dict(ctx=[40, 7, 300], batch=3, w_other=synth.W_Q5_K, w_down=synth.W_Q8_0, kv_dtype=synth.KV_F16),
    dict(ctx=[12, 0, 33, 64, 5, 17, 90, 2, 45, 9, 1, 60, 31, 16, 15, 200, 3, 8, 77, 50], batch=20,
         w_other=synth.W_Q8_0, w_down=synth.W_Q5_K, qk_norm=True, kv_dtype=synth.KV_Q8_0),
    dict(ctx=[40, 7], batch=2, ffn=8448, w_other=synth.W_Q8_0, w_down=synth.W_Q8_0),
    # Q6_K gate/up with SwiGLU on many tile pairs: 8 rows and a ragged 12, hidden 768 (three
    # super-blocks: 2-byte aligned Q6_K rows) and 1024 (16-byte aligned)
    # (gu: the gate/up launch the case must take, (tile loop?, batch tiles); 12 rows need
    # K of seven super-blocks for the tile loop, so hidden 768 takes split-K there)
    dict(ctx=[40, 7, 300, 0, 16, 90, 1, 33], batch=8, hidden=768, ffn=8192, w_other=synth.W_Q6_K,
         kv_dtype=synth.KV_F16, gu=(True, 1)),
    dict(ctx=[3, 70, 11, 0, 200, 15, 16, 17, 64, 5, 90, 31], batch=12, hidden=768, ffn=8448, w_other=synth.W_Q6_K,
         kv_dtype=synth.KV_Q8_0, qk_norm=True, gu=(False, 2)),
    dict(ctx=[9, 130, 47, 2, 61, 18, 77, 5, 100, 1], batch=10, hidden=2048, ffn=8192, w_other=synth.W_Q6_K,
         kv_dtype=synth.KV_F16, gu=(True, 2)),
    # Q4_K gate/up pairs at one batch tile: the whole-tile kernel (gu's third entry), one
    # wave per super-block: K = 4096 (528 pairs over 256 workgroups: two or three each), an
    # odd unit count per row (hidden 768), and K = 1024
    dict(ctx=[40, 7, 300, 0, 16, 90, 1, 33], batch=8, hidden=4096, ffn=8448, kv_dtype=synth.KV_F16,
         gu=(True, 1, True)),
    dict(ctx=[5, 64, 200, 17, 0], batch=5, hidden=768, ffn=8192, kv_dtype=synth.KV_Q8_0, qk_norm=True,
         gu=(True, 1, True)),
    dict(ctx=[31, 1], batch=2, hidden=1024, ffn=9216, gu=(True, 1, True)),
    # Q6_K down with its residual update at one batch tile: K-chunk staging (dn), K of 56
    # super-blocks (four stages of 14) and 48 (three of 16)
    dict(ctx=[40, 7, 300, 0, 16, 90, 1, 33], batch=8, ffn=14336, w_down=synth.W_Q6_K, kv_dtype=synth.KV_F16,
         dn=True),
    dict(ctx=[5, 64, 200], batch=3, ffn=12288, w_down=synth.W_Q6_K, qk_norm=True, dn=True),
    # Wo from 2048 to 4096 (256 tiles) at one batch tile: the whole-tile kernel's residual
    # update (wo), 16 query heads on 2 KV heads of 128
    dict(ctx=[60, 3, 250, 17, 0, 99], batch=6, hidden=4096, n_q_heads=16, n_kv_heads=2, head_dim=128, ffn=1024,
         kv_dtype=synth.KV_F16, wo=True),
    # 17 to 32 rows of Q4_K: the gate/up pairs on the row-block kernel (rb), K = 4096 in two
    # ranges, and at hidden 2048 in one (the epilogue straight from LDS); the other GEMMs
    # on the split-K kernel
    dict(ctx=[12, 0, 33, 64, 5, 17, 90, 2, 45, 9, 1, 60, 31, 16, 15, 200, 3, 8, 77, 50, 6, 140, 29, 11], batch=24,
         hidden=4096, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=1024, w_down=synth.W_Q4_K,
         kv_dtype=synth.KV_Q8_0, qk_norm=True, rb=True),
    dict(ctx=[(37 * i) % 301 for i in range(32)], batch=32, hidden=2048, n_q_heads=16, n_kv_heads=8, head_dim=128,
         ffn=4096, w_down=synth.W_Q4_K, kv_dtype=synth.KV_F16, rb=True),
]


def run_layer_case(torch, gr, orc, wl, ctx, layer=0):
    lw = synth.layer_weights(wl, layer)
    c = np.asarray(ctx, np.int32)
    kv = synth.kv_state(wl, c, n_layers=1)
    x = synth.input_x(wl, len(c))
    pm = kv.pages
    t, W = upload_layer(gr, torch, lw)
    kp, vp = dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch)
    xg = dev(x, torch)
    gr.gr_decode_layer(cfg_of(gr, wl), W, kp, vp, pm.num_pages, xg, dev(pm.block_table, torch), dev(c, torch),
                       int(c.max()))
    got = host(xg)
    okp, ovp = kv.k_pools[0].copy(), kv.v_pools[0].copy()
    want = orc.decode_layer(wl, lw, okp, ovp, x, pm.block_table, c)
    return got, want, (host(kp), host(vp)), (okp, ovp), kv


@pytest.mark.parametrize("case", range(len(LAYER_CASES)))
def test_tiny_layer_matches_oracle(torch, gr, orc, case):
    spec = dict(LAYER_CASES[case])
    ctx = spec.pop("ctx")
    gu = spec.pop("gu", None)
    dn = spec.pop("dn", None)
    wo = spec.pop("wo", None)
    rb = spec.pop("rb", None)
    wl = tiny(**spec)
    say("layer case", case, spec, ctx)
    if rb:  # the gate/up launch this case exists to cover
        sh = gr.gr_gemm_launch_shape(synth.W_Q4_K, wl.ffn, wl.hidden, len(ctx), gr.GEMM_EPI_SWIGLU)
        say("  gate/up launch", sh["kernel"])
        assert sh["row_block"]
    if gu is not None:
        # the gate/up kernel this case exists to cover (so the choice cannot drift unseen)
        sh = gr.gr_gemm_launch_shape(synth.layer_weights(wl, 0).tgate, wl.ffn, wl.hidden, len(ctx), gr.GEMM_EPI_SWIGLU)
        say("  gate/up launch", sh)
        assert (sh["tile_loop"], sh["btn"]) == gu[:2]
        if len(gu) > 2:
            assert sh["whole_tile"] == gu[2]
    if wo is not None:  # the Wo launch this case exists to cover
        sh = gr.gr_gemm_launch_shape(synth.layer_weights(wl, 0).to, wl.hidden, wl.n_q_heads * wl.head_dim, len(ctx),
                                     gr.GEMM_EPI_RESIDUAL)
        say("  Wo launch", sh)
        assert sh["whole_tile"] == wo
    if dn is not None:  # the down launch this case exists to cover
        sh = gr.gr_gemm_launch_shape(wl.w_down, wl.hidden, wl.ffn, len(ctx), gr.GEMM_EPI_RESIDUAL)
        say("  down launch", sh)
        assert sh["k_chunks"] == dn
    got, want, gpools, opools, kv = run_layer_case(torch, gr, orc, wl, ctx)
    assert np.isfinite(got).all()
    err, rerr = rel_l2(got, want), row_rel_l2(got, want)
    say("  rel_l2", err, "worst row", rerr)
    assert err <= tol(wl.kv_dtype) and rerr <= tol(wl.kv_dtype)
    # the appended token: every row's new K and V decode close to the oracle's stored token
    c = np.asarray(ctx, np.int32)
    n_tok = c + 1
    for i, is_v in enumerate((False, True)):
        g = orc.gather_kv(gpools[i], wl.kv_dtype, is_v, wl.n_kv_heads, wl.head_dim, kv.pages.block_table, n_tok)
        o = orc.gather_kv(opools[i], wl.kv_dtype, is_v, wl.n_kv_heads, wl.head_dim, kv.pages.block_table, n_tok)
        assert np.isfinite(g).all()
        # the new token of each row on its own (not diluted by the untouched context),
        # and tokens before it unchanged
        off = 0
        for n in n_tok:
            assert rel_l2(g[off + n - 1], o[off + n - 1]) <= tol(wl.kv_dtype)
            assert np.array_equal(g[off:off + n - 1], o[off:off + n - 1])
            off += n


def test_layer_batched_matches_rows_alone(torch, gr, orc):
    wl = tiny(batch=4, kv_dtype=synth.KV_F16, qk_norm=True)
    ctx = [7, 100, 16, 50]
    lw = synth.layer_weights(wl, 0)
    c = np.asarray(ctx, np.int32)
    kv = synth.kv_state(wl, c, n_layers=1)
    x = synth.input_x(wl, 4)
    t, W = upload_layer(gr, torch, lw)
    cfg = cfg_of(gr, wl)
    bt = kv.pages.block_table

    def run(rows):
        kp, vp = dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch)
        xg = dev(x[rows], torch)
        gr.gr_decode_layer(cfg, W, kp, vp, kv.pages.num_pages, xg, dev(bt[rows], torch), dev(c[rows], torch),
                           int(c.max()))
        return host(xg)

    full = run([0, 1, 2, 3])
    for r in range(4):
        assert rel_l2(run([r])[0], full[r]) <= 1e-5
    # rows leaving and joining between steps: a subset in another order
    sub = run([3, 1])
    assert rel_l2(sub, full[[3, 1]]) <= 1e-5


def test_qwen3_0p6b_stack_matches_oracle(torch, gr, orc):
    """Qwen3-0.6B-shaped stack, 28 layers, B=8, f16 KV, QK-norm: every layer output."""
    wl = synth.WORKLOADS["qwen3_0p6b"]
    c = synth.ctx_lens(wl)
    kv = synth.kv_state(wl, c)
    x = synth.input_x(wl)
    pm = kv.pages
    cfg = cfg_of(gr, wl)
    xg = dev(x, torch)
    bt, cg = dev(pm.block_table, torch), dev(c, torch)
    cur = x
    worst = 0.0
    ws = gr.workspace(gr.decode_layer_workspace_size(cfg, wl.batch, int(c.max())))
    for layer in range(wl.n_layers):
        lw = synth.layer_weights(wl, layer)
        t, W = upload_layer(gr, torch, lw)
        kp, vp = dev(kv.k_pools[layer], torch), dev(kv.v_pools[layer], torch)
        gr.gr_decode_layer(cfg, W, kp, vp, pm.num_pages, xg, bt, cg, int(c.max()), ws=ws)
        okp, ovp = kv.k_pools[layer].copy(), kv.v_pools[layer].copy()
        cur = orc.decode_layer(wl, lw, okp, ovp, cur, pm.block_table, c)
        err, rerr = rel_l2(host(xg), cur), row_rel_l2(host(xg), cur)
        worst = max(worst, rerr)
        say(f"  layer {layer}: rel_l2 {err:.3e}, worst row {rerr:.3e}")
        assert err <= tol(wl.kv_dtype) and rerr <= tol(wl.kv_dtype), layer
    say("worst", worst)
