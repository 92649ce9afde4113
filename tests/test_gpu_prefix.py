"""Shared prefix pages (aliased block-table entries) on the GPU, against the fp64 oracle.

Sequences that share a prompt prefix point their first block-table entries at the same
physical pages (only full pages are shared; each sequence's own tokens, and the slot the
step appends into, sit in its private pages).  The kernels address pages only through the
block table, so sharing needs no kernel of its own: the step must equal the oracle's and
leave the shared pages' bytes untouched.
"""
import dataclasses

import numpy as np
import pytest

import synth
from gpu_util import dev, host, rel_l2, say, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


@pytest.fixture(scope="module")
def gr():
    import continuous_quantized_decode_amd as gr
    gr.lib()
    return gr


def _share_prefix(kv, rows, n_shared):
    """Point the first n_shared block-table entries of `rows` at row 0's pages."""
    bt = kv.pages.block_table.copy()
    for r in rows:
        bt[r, :n_shared] = bt[0, :n_shared]
    return bt


def _upload(gr, torch, lw):
    t = {k: dev(getattr(lw, k), torch) for k in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up",
                                                  "w_down")}
    if lw.q_norm is not None:
        t["q_norm"] = dev(lw.q_norm, torch)
        t["k_norm"] = dev(lw.k_norm, torch)
    for k in ("tq", "tk", "tv", "to", "tgate", "tup", "tdown"):
        t[k] = getattr(lw, k)
    return t, gr.layer_weights(t)


@pytest.mark.parametrize("kv_dtype", [synth.KV_F16, synth.KV_Q8_0])
def test_decode_layer_with_shared_prefix_pages(torch, gr, orc, kv_dtype):
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_0p6b"], n_layers=1, kv_dtype=kv_dtype)
    ctx = np.array([200, 170, 333, 129], np.int32)  # every row holds at least 8 full pages
    kv = synth.kv_state(wl, ctx, n_layers=1)
    shared = 8
    bt = _share_prefix(kv, [1, 2, 3], shared)
    shared_pages = bt[0, :shared]
    lw = synth.layer_weights(wl, 0)
    t, w = _upload(gr, torch, lw)
    cfg = gr.layer_cfg(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.ffn, wl.rms_eps, wl.rope_theta,
                       wl.rope_style, wl.qk_norm, wl.kv_dtype)
    x = synth.input_x(wl, len(ctx))
    kp, vp = dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch)
    xg = dev(x, torch)
    say("shared prefix decode layer kv", kv_dtype)
    gr.gr_decode_layer(cfg, w, kp, vp, kv.pages.num_pages, xg, dev(bt, torch), dev(ctx, torch), int(ctx.max()))
    torch.cuda.synchronize()
    okp, ovp = kv.k_pools[0].copy(), kv.v_pools[0].copy()
    want = orc.decode_layer(wl, lw, okp, ovp, x, bt, ctx)
    err = rel_l2(host(xg), want)
    say(f"  rel_l2 {err:.3e}")
    assert err <= (5e-3 if kv_dtype == synth.KV_Q8_0 else 2e-3)
    for got, orig in ((host(kp), kv.k_pools[0]), (host(vp), kv.v_pools[0])):
        np.testing.assert_array_equal(got[shared_pages], orig[shared_pages])


def test_prompt_chunks_after_a_shared_prefix(torch, gr, orc):
    """Two sequences share a 64-token prefix; each continues its own prompt in one mixed step."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=2, kv_dtype=synth.KV_F16, qk_norm=True)
    ctx = np.array([64, 64, 90], np.int32)
    kv = synth.kv_state(wl, ctx, n_layers=2, extra_slot=12)
    bt = _share_prefix(kv, [1], 4)
    layers = [synth.layer_weights(wl, layer) for layer in range(2)]
    keep, ws = [], []
    for lw in layers:
        tt, w = _upload(gr, torch, lw)
        keep.append(tt)
        ws.append(w)
    cfg = gr.layer_cfg(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.ffn, wl.rms_eps, wl.rope_theta,
                       wl.rope_style, wl.qk_norm, wl.kv_dtype)
    kd = [dev(p, torch) for p in kv.k_pools]
    vd = [dev(p, torch) for p in kv.v_pools]
    args = gr.StackArgs(cfg, ws, kd, vd)
    seq = np.array([0] * 12 + [1] * 7 + [2], np.int32)
    pos = np.concatenate([64 + np.arange(12), 64 + np.arange(7), [90]]).astype(np.int32)
    x = synth.activations(np.random.default_rng(6), len(seq), wl.hidden)
    xg = dev(x, torch)
    gr.gr_mixed_stack(args, kv.pages.num_pages, xg, dev(bt, torch), dev(seq, torch), dev(pos, torch), int(pos.max()))
    torch.cuda.synchronize()
    ok = [p.copy() for p in kv.k_pools]
    ov = [p.copy() for p in kv.v_pools]
    outs, _ = orc.mixed_stack(wl, layers, ok, ov, x, bt, seq, pos)
    err = rel_l2(host(xg), outs[-1])
    say(f"shared prefix mixed step rel_l2 {err:.3e}")
    assert err <= 2e-3
    for layer in range(2):
        np.testing.assert_array_equal(host(kd[layer])[bt[0, :4]], kv.k_pools[layer][bt[0, :4]])
