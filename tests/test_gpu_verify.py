"""GPU parity of the speculative verification step (gr_verify_stack, gr_spec_accept) against
the fp64 oracle, through the C ABI.

T tokens per sequence go through the stack in one step; the oracle runs them layer by layer,
token by token (equal to T decode steps).  Bars as for decode layers: relative L2 over each
output ≤ 2e-3 for f32 / f16 KV, 5e-3 for q8_0 KV; the pools' stored tokens are compared
after decoding them; acceptance is bit-exact.
"""
import dataclasses

import numpy as np
import pytest

import synth
from gpu_util import dev, host, rel_l2, say, torch_cuda

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


def _upload(gr, torch, lw):
    t = {k: dev(getattr(lw, k), torch) for k in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up",
                                                  "w_down")}
    if lw.q_norm is not None:
        t["q_norm"] = dev(lw.q_norm, torch)
        t["k_norm"] = dev(lw.k_norm, torch)
    for k in ("tq", "tk", "tv", "to", "tgate", "tup", "tdown"):
        t[k] = getattr(lw, k)
    return t, gr.layer_weights(t)


def _cfg(gr, wl):
    return gr.layer_cfg(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.ffn, wl.rms_eps, wl.rope_theta,
                        wl.rope_style, wl.qk_norm, wl.kv_dtype)


def _run(torch, gr, orc, wl, ctx, t, n_layers, with_head, seed=0):
    ctx = np.asarray(ctx, np.int32)
    b = len(ctx)
    kv = synth.kv_state(wl, ctx, n_layers=n_layers, extra_slot=t)
    pm = kv.pages
    layers = [synth.layer_weights(wl, layer) for layer in range(n_layers)]
    x = synth.activations(np.random.default_rng(900 + seed), b * t, wl.hidden)
    head = synth.head_weights(wl) if with_head else None
    keep, ws = [], []
    for lw in layers:
        tt, w = _upload(gr, torch, lw)
        keep.append(tt)
        ws.append(w)
    kd = [dev(p, torch) for p in kv.k_pools]
    vd = [dev(p, torch) for p in kv.v_pools]
    args = gr.StackArgs(_cfg(gr, wl), ws, kd, vd)
    xg = dev(x, torch)
    logits = None
    hn = hw = None
    if head is not None:
        hn, hw = dev(head[0], torch), dev(head[1], torch)
        logits = torch.empty((b * t, wl.vocab), dtype=torch.float32, device="cuda")
    say("verify", wl.name, "ctx", ctx.tolist(), "T", t, "layers", n_layers, "kv", wl.kv_dtype)
    gr.gr_verify_stack(args, pm.num_pages, xg, dev(pm.block_table, torch), dev(ctx, torch), int(ctx.max()), t,
                       head_norm=hn, head_w=hw, head_wtype=wl.w_head, vocab=wl.vocab if head is not None else 0,
                       logits=logits)
    torch.cuda.synchronize()
    okp = [p.copy() for p in kv.k_pools]
    ovp = [p.copy() for p in kv.v_pools]
    outs, want_logits = orc.verify_stack(wl, layers, okp, ovp, x, pm.block_table, ctx, t, head=head)
    err = rel_l2(host(xg), outs[-1])
    say(f"  rel_l2 x {err:.3e}")
    assert err <= tol(wl.kv_dtype)
    if head is not None:
        lerr = rel_l2(host(logits), want_logits)
        say(f"  rel_l2 logits {lerr:.3e}")
        assert lerr <= tol(wl.kv_dtype)
    # the step's K/V landed at every token's position (decoded, for the last layer)
    n_tok = ctx + t
    starts = np.concatenate([[0], np.cumsum(n_tok)[:-1]])
    for is_v, got_pool, want_pool in ((False, kd[-1], okp[-1]), (True, vd[-1], ovp[-1])):
        g = orc.gather_kv(host(got_pool), wl.kv_dtype, is_v, wl.n_kv_heads, wl.head_dim, pm.block_table, n_tok)
        w = orc.gather_kv(want_pool, wl.kv_dtype, is_v, wl.n_kv_heads, wl.head_dim, pm.block_table, n_tok)
        for r in range(b):
            sl = slice(int(starts[r] + ctx[r]), int(starts[r] + ctx[r] + t))
            assert rel_l2(g[sl], w[sl]) <= tol(wl.kv_dtype)
    return host(xg), (host(logits) if logits is not None else None)


CASES = [
    dict(name="tiny f32", wl=dict(), ctx=[5, 31, 16], t=3),
    dict(name="tiny f16 qk", wl=dict(kv_dtype=synth.KV_F16, qk_norm=True), ctx=[0, 15, 47, 100], t=4),
    dict(name="tiny q8_0 norm-rope", wl=dict(kv_dtype=synth.KV_Q8_0, rope_style=synth.ROPE_NORM), ctx=[14, 60], t=5),
    dict(name="tiny D128 q8_0", wl=dict(kv_dtype=synth.KV_Q8_0, head_dim=128, n_q_heads=4, n_kv_heads=1),
         ctx=[200, 3, 33], t=8),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_verify_layers_match_oracle(torch, gr, orc, case):
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=2, **case["wl"])
    _run(torch, gr, orc, wl, case["ctx"], case["t"], 2, with_head=False)


def test_verify_one_token_equals_decode(torch, gr, orc):
    """T = 1 takes the decode step's own launches: bitwise equal outputs."""
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_0p6b"], n_layers=2)
    ctx = np.array([40, 300, 7, 129], np.int32)
    kv = synth.kv_state(wl, ctx, n_layers=2)
    pm = kv.pages
    layers = [synth.layer_weights(wl, layer) for layer in range(2)]
    keep, ws = [], []
    for lw in layers:
        tt, w = _upload(gr, torch, lw)
        keep.append(tt)
        ws.append(w)
    x = synth.input_x(wl, len(ctx))
    outs = []
    for fn in ("gr_decode_stack", "gr_verify_stack"):
        kd = [dev(p, torch) for p in kv.k_pools]
        vd = [dev(p, torch) for p in kv.v_pools]
        args = gr.StackArgs(_cfg(gr, wl), ws, kd, vd)
        xg = dev(x, torch)
        if fn == "gr_decode_stack":
            gr.gr_decode_stack(args, pm.num_pages, xg, dev(pm.block_table, torch), dev(ctx, torch), int(ctx.max()))
        else:
            gr.gr_verify_stack(args, pm.num_pages, xg, dev(pm.block_table, torch), dev(ctx, torch), int(ctx.max()), 1)
        torch.cuda.synchronize()
        outs.append(host(xg))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_decode_stack_repeats_bitwise(torch, gr):
    """The same step twice gives the same bits: every cross-workgroup sum (the RMSNorm
    statistics, the attention partial states) is added in a fixed order or exactly."""
    wl = dataclasses.replace(synth.WORKLOADS["llama3_8b"], n_layers=2)
    ctx = synth.ctx_lens(wl)
    kv = synth.kv_state(wl, ctx, n_layers=2)
    pm = kv.pages
    layers = [synth.layer_weights(wl, layer) for layer in range(2)]
    keep, ws = [], []
    for lw in layers:
        tt, w = _upload(gr, torch, lw)
        keep.append(tt)
        ws.append(w)
    x = synth.input_x(wl, len(ctx))
    outs = []
    for rep in range(3):
        kd = [dev(p, torch) for p in kv.k_pools]
        vd = [dev(p, torch) for p in kv.v_pools]
        xg = dev(x, torch)
        gr.gr_decode_stack(gr.StackArgs(_cfg(gr, wl), ws, kd, vd), pm.num_pages, xg, dev(pm.block_table, torch),
                           dev(ctx, torch), int(ctx.max()))
        torch.cuda.synchronize()
        outs.append((host(xg), host(kd[1]), host(vd[1])))
    for rep in (1, 2):
        for a, b in zip(outs[0], outs[rep]):
            np.testing.assert_array_equal(a, b)


def test_verify_qwen3_0p6b_shapes(torch, gr, orc):
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_0p6b"], n_layers=3)
    _run(torch, gr, orc, wl, [64, 1000, 255, 17], 4, 3, with_head=False, seed=1)


def test_verify_llama3_layers_and_head(torch, gr, orc):
    """Llama-3-8B shapes at B = 8, T = 5 (40 rows through every GEMM) with the output head."""
    wl = synth.WORKLOADS["llama3_8b"]
    ctx = synth.ctx_lens(wl)
    _run(torch, gr, orc, wl, ctx, 5, 2, with_head=True, seed=2)


def test_verify_llama3_t2_one_layer_and_head(torch, gr, orc):
    """bench.py's verification shape (Llama-3-8B, B = 8, T = 2: 16 rows), one layer and the
    head: gate/up and the head take the tile loop with two batch tiles."""
    wl = dataclasses.replace(synth.WORKLOADS["llama3_8b"], n_layers=1)
    assert gr.gr_gemm_launch_shape(wl.w_head, wl.vocab, wl.hidden, 16)["btn"] == 2
    _run(torch, gr, orc, wl, synth.ctx_lens(wl), 2, 1, with_head=True, seed=6)


def test_spec_accept_matches_oracle(torch, gr, orc):
    rng = np.random.default_rng(3)
    b, t = 37, 6
    draft = rng.integers(0, 4, (b, t)).astype(np.int32)
    sampled = rng.integers(0, 4, (b, t)).astype(np.int32)
    sampled[::3, :t - 1] = draft[::3, 1:]  # some rows accept everything
    got = host(gr.gr_spec_accept(dev(sampled, torch), dev(draft, torch)))
    np.testing.assert_array_equal(got, orc.spec_accept(sampled, draft))
    assert (got[::3] == t - 1).all()


def test_verify_then_sample_then_accept(torch, gr, orc):
    """The verification chain on the GPU: logits of every position, one draw per position,
    acceptance; draws and acceptance equal the oracle's on the same logits."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=2, vocab=1000, kv_dtype=synth.KV_F16)
    t = 4
    ctx = np.array([20, 50, 3], np.int32)
    _, logits = _run(torch, gr, orc, wl, ctx, t, 2, with_head=True, seed=4)
    rng = np.random.default_rng(5)
    u = synth.sample_uniforms(rng, len(ctx) * t)
    lg = dev(logits, torch)
    sampled = host(gr.gr_sample(lg, gr.sample_params(0.8, 0.95, 40, u, b=len(u)))).reshape(len(ctx), t)
    np.testing.assert_array_equal(sampled.reshape(-1), orc.sample(logits, 0.8, 0.95, 40, u))
    draft = np.concatenate([np.full((len(ctx), 1), 1, np.int32), sampled[:, :t - 1]], axis=1)
    draft[1, 2] = (draft[1, 2] + 1) % 1000  # the second row's second proposal is wrong
    got = host(gr.gr_spec_accept(dev(sampled.astype(np.int32), torch), dev(draft, torch)))
    np.testing.assert_array_equal(got, orc.spec_accept(sampled, draft))
    assert got.tolist() == [t - 1, 1, t - 1]
