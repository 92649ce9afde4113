"""GPU parity of steps with more than 64 rows (the 2-D tiled many-row GEMM) against the
fp64 oracle, through the C ABI.

Prompt chunks of a few hundred tokens (Leone, "What ships": chunked prefill; chunks of
256 tokens within a 512-token step budget) put hundreds of rows through every GEMM of a
layer.  Bars: relative L2 <= 1e-4 for a GEMM or head alone (the skinny kernels' bar: the
same exact bf16 hi/lo products with fp32 sums), and the layer bars (2e-3 for f32 / f16
KV, 5e-3 for q8_0 KV) for layers and steps.
"""
import dataclasses

import numpy as np
import pytest

import synth
from gpu_util import dev, host, rel_l2, say, torch_cuda
from test_gpu_mixed import Session, _mixed_rows

pytestmark = pytest.mark.gpu

KERNEL_TOL = 1e-4


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


GEMM_CASES = [
    (synth.W_Q4_K, 65, 200, 1024),     # one row past the skinny kernels, ragged tiles
    (synth.W_Q4_K, 100, 4096, 4096),
    (synth.W_Q4_K, 257, 300, 2048),    # ragged activation tile group
    (synth.W_Q4_K, 512, 1000, 4096),   # the largest step
    (synth.W_Q4_K, 96, 16, 256),       # one weight tile, one super-block (no K split)
    (synth.W_Q4_K, 300, 9000, 1024),   # wider than the K-split limit
    (synth.W_Q6_K, 72, 64, 2048),      # 16-byte aligned rows
    (synth.W_Q6_K, 129, 500, 3072),    # 2-byte aligned rows (12 super-blocks)
    (synth.W_Q6_K, 300, 700, 768),     # odd super-blocks per row
    (synth.W_Q6_K, 512, 512, 14336),   # Llama-3-8B down K
]


@pytest.mark.parametrize("wtype,b,n,k", GEMM_CASES)
def test_many_row_gemm_matches_oracle(torch, gr, orc, wtype, b, n, k):
    rng = np.random.default_rng(2000 + b + n + k)
    w = synth.weight(rng, wtype, n, k)
    x = rng.standard_normal((b, k), dtype=np.float32)
    shape = gr.gr_gemm_launch_shape(wtype, n, k, b)
    say("many-row gemm", wtype, b, n, k, shape)
    assert shape["many_rows"]
    fn = gr.gr_q4k_gemm if wtype == synth.W_Q4_K else gr.gr_q6k_gemm
    got = host(fn(dev(w, torch), dev(x, torch), n))
    err = rel_l2(got, orc.gemm(wtype, w, x, n, k))
    say("  rel_l2", err)
    assert err <= KERNEL_TOL


def test_many_row_gemm_rows_independent(torch, gr):
    """Rows computed among 300 equal the same rows computed among 8 (skinny kernel) and
    alone, to fp32 rounding."""
    rng = np.random.default_rng(9)
    n, k = 256, 2048
    w = dev(synth.q4k_weight(rng, n, k), torch)
    x = rng.standard_normal((300, k), dtype=np.float32)
    full = host(gr.gr_q4k_gemm(w, dev(x, torch), n))
    few = host(gr.gr_q4k_gemm(w, dev(x[290:298], torch), n))
    assert rel_l2(full[290:298], few) <= 1e-6
    one = host(gr.gr_q4k_gemm(w, dev(x[7:8], torch), n))
    assert rel_l2(full[7:8], one) <= 1e-6


@pytest.mark.parametrize("wtype", [synth.W_Q4_K, synth.W_Q6_K])
def test_many_row_output_head(torch, gr, orc, wtype):
    rng = np.random.default_rng(31 + wtype)
    h, vocab, b = 1024, 3000, 130
    x = synth.activations(rng, b, h)
    norm = (1.0 + 0.1 * rng.standard_normal(h)).astype(np.float32)
    w = synth.weight(rng, wtype, vocab, h)
    got = host(gr.gr_output_head(dev(x, torch), dev(norm, torch), 1e-6, dev(w, torch), wtype, vocab))
    err = rel_l2(got, orc.output_head(x, norm, 1e-6, w, wtype, vocab))
    say("many-row head", wtype, b, f"rel_l2 {err:.3e}")
    assert err <= KERNEL_TOL


def test_q5_q8_rows_above_64_are_refused(torch, gr):
    rng = np.random.default_rng(3)
    w = dev(synth.weight(rng, synth.W_Q8_0, 32, 256), torch)
    x = dev(rng.standard_normal((65, 256), dtype=np.float32), torch)
    with pytest.raises(RuntimeError):
        gr.gr_q8_0_gemm(w, x, 32)


def _upload(gr, torch, lw):
    t = {k: dev(getattr(lw, k), torch) for k in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up",
                                                  "w_down")}
    if lw.q_norm is not None:
        t["q_norm"] = dev(lw.q_norm, torch)
        t["k_norm"] = dev(lw.k_norm, torch)
    for k in ("tq", "tk", "tv", "to", "tgate", "tup", "tdown"):
        t[k] = getattr(lw, k)
    return t, gr.layer_weights(t)


@pytest.mark.parametrize("wl_name,batch,rep", [
    ("tiny", 100, dict(kv_dtype=synth.KV_F16, qk_norm=True)),
    ("tiny", 200, dict(kv_dtype=synth.KV_Q8_0, w_other=synth.W_Q6_K, w_down=synth.W_Q4_K)),
    ("qwen3_0p6b", 80, dict()),
])
def test_many_row_decode_layer(torch, gr, orc, wl_name, batch, rep):
    """A decode layer with 80-200 rows: every GEMM (QKV store, Wo and down residual with
    their packs and norm sums, gate/up SwiGLU) in the many-row kernel."""
    wl = dataclasses.replace(synth.WORKLOADS[wl_name], batch=batch, **rep)
    c = synth.ctx_lens(wl)
    kv = synth.kv_state(wl, c, n_layers=1)
    lw = synth.layer_weights(wl, 0)
    x = synth.input_x(wl, batch)
    t, W = _upload(gr, torch, lw)
    kp, vp = dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch)
    xg = dev(x, torch)
    cfg = gr.layer_cfg(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.ffn, wl.rms_eps, wl.rope_theta,
                       wl.rope_style, wl.qk_norm, wl.kv_dtype)
    say("many-row layer", wl_name, batch, rep)
    gr.gr_decode_layer(cfg, W, kp, vp, kv.pages.num_pages, xg, dev(kv.pages.block_table, torch), dev(c, torch),
                       int(c.max()))
    okp, ovp = kv.k_pools[0].copy(), kv.v_pools[0].copy()
    want = orc.decode_layer(wl, lw, okp, ovp, x, kv.pages.block_table, c)
    err = rel_l2(host(xg), want)
    say(f"  rel_l2 {err:.3e}")
    assert err <= tol(wl.kv_dtype)


def test_prefill_chunk_256_with_decode_rows(torch, gr, orc):
    """A 256-token prompt chunk resuming a 40-token prefix, next to eight decode rows
    (264 rows; Qwen3-0.6B shapes, two layers)."""
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_0p6b"], n_layers=2)
    ctx = np.array([40, 500, 77, 1200, 9, 300, 64, 128, 1], np.int32)
    s = Session(torch, gr, orc, wl, ctx, 256, False)
    rng = np.random.default_rng(10)
    seq, pos = _mixed_rows(rng, ctx, [256] + [1] * 8)
    x = synth.activations(rng, len(seq), wl.hidden)
    s.step(x, seq, pos, "qwen3 256-token chunk + 8 decode")


def test_two_chunks_fill_the_512_budget_with_head(torch, gr, orc):
    """Two prompt chunks (256 from an empty cache, 248 resuming) and eight decode rows:
    512 rows, with the output head (tiny shapes, vocab 1000)."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=2, kv_dtype=synth.KV_F16, vocab=1000)
    ctx = np.array([0, 100, 5, 60, 300, 17, 250, 33, 90, 2], np.int32)
    s = Session(torch, gr, orc, wl, ctx, 256, True)
    rng = np.random.default_rng(11)
    seq, pos = _mixed_rows(rng, ctx, [256, 248] + [1] * 8)
    x = synth.activations(rng, len(seq), wl.hidden)
    s.step(x, seq, pos, "tiny 512 rows")


def test_head_on_selected_rows(torch, gr, orc):
    """The head on the rows that need logits only (each chunk's last token and the decode
    rows): equal to those rows of the all-rows logits.  A repeated index is allowed."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=2, kv_dtype=synth.KV_F16, vocab=1000)
    ctx = np.array([0, 100, 5, 60, 300, 17, 250, 33, 90, 2], np.int32)
    s = Session(torch, gr, orc, wl, ctx, 200, True)
    rng = np.random.default_rng(12)
    seq, pos = _mixed_rows(rng, ctx, [200, 100] + [1] * 8)
    need = [int(np.nonzero((seq == 0) & (pos == 199))[0][0]), int(np.nonzero((seq == 1) & (pos == 199))[0][0])]
    need += [int(i) for i in np.nonzero(seq >= 2)[0]] + [need[0]]
    x = synth.activations(rng, len(seq), wl.hidden)
    s.step(x, seq, pos, "tiny 308 rows, head on 11", head_rows=need)


@pytest.mark.parametrize("kv_dtype", [synth.KV_F32, synth.KV_F16, synth.KV_Q8_0])
def test_contiguous_chunk_rows_share_page_reads(torch, gr, orc, kv_dtype):
    """Rows in sequence order (a chunk's rows next to each other, as a scheduler lays them
    out): the standalone attention takes 8 / (Hq / Hkv) consecutive rows of one sequence to
    a wave.  Chunks of odd lengths, resumed mid-page and from an empty cache, so groups
    straddle sequence boundaries and rows end on different pages of a split."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=2, kv_dtype=kv_dtype, qk_norm=True)
    ctx = np.array([0, 37, 300, 5, 64, 1], np.int32)
    s = Session(torch, gr, orc, wl, ctx, 70, False)
    spec = [70, 33, 1, 7, 50, 3]
    seq = np.concatenate([np.full(n, i) for i, n in enumerate(spec)]).astype(np.int32)
    pos = np.concatenate([ctx[i] + np.arange(n) for i, n in enumerate(spec)]).astype(np.int32)
    x = synth.activations(np.random.default_rng(13 + kv_dtype), len(seq), wl.hidden)
    s.step(x, seq, pos, f"contiguous rows kv={kv_dtype}")


def test_contiguous_chunk_rows_llama_heads(torch, gr, orc):
    """The same with Llama-3-style grouped heads (Hq / Hkv = 4: two rows to a wave) and
    head_dim 128, f16 KV, with the head on the chunks' last tokens."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=1, kv_dtype=synth.KV_F16, head_dim=128,
                             n_q_heads=8, n_kv_heads=2, vocab=500)
    ctx = np.array([0, 200, 17], np.int32)
    s = Session(torch, gr, orc, wl, ctx, 90, True)
    spec = [90, 41, 1]
    seq = np.concatenate([np.full(n, i) for i, n in enumerate(spec)]).astype(np.int32)
    pos = np.concatenate([ctx[i] + np.arange(n) for i, n in enumerate(spec)]).astype(np.int32)
    x = synth.activations(np.random.default_rng(17), len(seq), wl.hidden)
    s.step(x, seq, pos, "contiguous rows, 4 q heads per kv head", head_rows=[89, 130, 131])
