"""GPU parity of the mixed step (gr_mixed_stack) against the fp64 oracle, through the C ABI.

Rows are placed by (sequence, position): decode rows, verification runs and prompt chunks
(from an empty cache or resuming one) share one step, in shuffled row order.  Bars as for
decode layers: relative L2 ≤ 2e-3 for f32 / f16 KV, 5e-3 for q8_0 KV.
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


class Session:
    """Weights and pools on both sides; steps run on the GPU and in the oracle side by side."""

    def __init__(self, torch, gr, orc, wl, ctx, extra, with_head):
        self.torch, self.gr, self.orc, self.wl = torch, gr, orc, wl
        ctx = np.asarray(ctx, np.int32)
        kv = synth.kv_state(wl, ctx, n_layers=wl.n_layers, extra_slot=extra)
        self.pm = kv.pages
        self.layers = [synth.layer_weights(wl, layer) for layer in range(wl.n_layers)]
        self.keep, ws = [], []
        for lw in self.layers:
            tt, w = _upload(gr, torch, lw)
            self.keep.append(tt)
            ws.append(w)
        self.kd = [dev(p, torch) for p in kv.k_pools]
        self.vd = [dev(p, torch) for p in kv.v_pools]
        self.ok = [p.copy() for p in kv.k_pools]
        self.ov = [p.copy() for p in kv.v_pools]
        self.args = gr.StackArgs(_cfg(gr, wl), ws, self.kd, self.vd)
        self.bt = dev(self.pm.block_table, torch)
        self.head = synth.head_weights(wl) if with_head else None
        self.hd = (dev(self.head[0], torch), dev(self.head[1], torch)) if with_head else (None, None)

    def step(self, x, seq, pos, label, head_rows=None):
        torch, gr, wl = self.torch, self.gr, self.wl
        seq = np.asarray(seq, np.int32)
        pos = np.asarray(pos, np.int32)
        xg = dev(x, torch)
        logits = None
        if self.head is not None:
            n_logit = len(seq) if head_rows is None else len(head_rows)
            logits = torch.empty((n_logit, wl.vocab), dtype=torch.float32, device="cuda")
        say("mixed", label, "rows", len(seq))
        hr = None if head_rows is None else dev(np.asarray(head_rows, np.int32), torch)
        gr.gr_mixed_stack(self.args, self.pm.num_pages, xg, self.bt, dev(seq, torch), dev(pos, torch), int(pos.max()),
                          head_norm=self.hd[0], head_w=self.hd[1], head_wtype=wl.w_head,
                          vocab=wl.vocab if self.head is not None else 0, logits=logits, head_rows=hr)
        torch.cuda.synchronize()
        outs, want_logits = self.orc.mixed_stack(wl, self.layers, self.ok, self.ov, x, self.pm.block_table, seq, pos,
                                                 head=self.head)
        err = rel_l2(host(xg), outs[-1])
        say(f"  rel_l2 x {err:.3e}")
        assert err <= tol(wl.kv_dtype), label
        if logits is not None:
            if head_rows is not None:
                want_logits = want_logits[np.asarray(head_rows)]
            lerr = rel_l2(host(logits), want_logits)
            say(f"  rel_l2 logits {lerr:.3e}")
            assert lerr <= tol(wl.kv_dtype), label


def _mixed_rows(rng, ctx, spec):
    """spec: per sequence the number of new tokens; rows shuffled."""
    seq = np.concatenate([np.full(n, s) for s, n in enumerate(spec)]).astype(np.int32)
    pos = np.concatenate([ctx[s] + np.arange(n) for s, n in enumerate(spec)]).astype(np.int32)
    perm = rng.permutation(len(seq))
    return seq[perm], pos[perm]


@pytest.mark.parametrize("kv_dtype", [synth.KV_F32, synth.KV_F16, synth.KV_Q8_0])
def test_mixed_step_tiny(torch, gr, orc, kv_dtype):
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=2, kv_dtype=kv_dtype, qk_norm=True)
    ctx = np.array([0, 300, 100, 64, 31], np.int32)
    s = Session(torch, gr, orc, wl, ctx, 24, False)
    rng = np.random.default_rng(kv_dtype)
    # a prompt chunk from an empty cache, a decode row, a resumed chunk, a verification run
    seq, pos = _mixed_rows(rng, ctx, [24, 1, 16, 4, 1])
    x = synth.activations(rng, len(seq), wl.hidden)
    s.step(x, seq, pos, f"tiny kv={kv_dtype}")


def test_prompt_in_chunks_with_decode_rows(torch, gr, orc):
    """A 100-token prompt from an empty cache in chunks of 40, 40 and 20, next to three
    sequences decoding one token per step (Qwen3-0.6B shapes)."""
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_0p6b"], n_layers=2)
    ctx = np.array([0, 500, 77, 1200], np.int32)
    s = Session(torch, gr, orc, wl, ctx, 100, False)
    rng = np.random.default_rng(7)
    done = 0
    for step, n in enumerate([40, 40, 20]):
        seq = np.concatenate([np.zeros(n, np.int32), np.array([1, 2, 3], np.int32)])
        pos = np.concatenate([np.arange(done, done + n), ctx[1:] + step]).astype(np.int32)
        perm = rng.permutation(len(seq))
        x = synth.activations(rng, len(seq), wl.hidden)
        s.step(x[perm], seq[perm], pos[perm], f"chunk {step}")
        done += n


def test_mixed_step_llama3_with_head(torch, gr, orc):
    """Llama-3-8B shapes: eight decode rows and a 56-token prompt chunk (64 rows) plus the head."""
    wl = dataclasses.replace(synth.WORKLOADS["llama3_8b"], n_layers=2)
    ctx = np.concatenate([synth.ctx_lens(wl), [0]]).astype(np.int32)
    s = Session(torch, gr, orc, wl, ctx, 56, True)
    rng = np.random.default_rng(8)
    seq, pos = _mixed_rows(rng, ctx, [1] * 8 + [56])
    x = synth.activations(rng, len(seq), wl.hidden)
    s.step(x, seq, pos, "llama3 8 decode + 56 prefill")
