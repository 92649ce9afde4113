"""Pins of the oracle's mixed step (no GPU): rows placed by (sequence, position), so decode
rows, verification runs and prompt chunks share one step (Leone, "What ships": chunked
prefill, continuous decode batching).  Its oracle runs the rows one at a time in position
order; the pins tie it to the decode and verification oracles and to chunking itself.
"""
import dataclasses

import numpy as np

import synth


def _wl(**kw):
    return dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=2, kv_dtype=synth.KV_F16, qk_norm=True, **kw)


def _state(wl, ctx, extra):
    kv = synth.kv_state(wl, np.asarray(ctx, np.int32), n_layers=wl.n_layers, extra_slot=extra)
    layers = [synth.layer_weights(wl, layer) for layer in range(wl.n_layers)]
    return kv, layers


def _pools(kv):
    return [p.copy() for p in kv.k_pools], [p.copy() for p in kv.v_pools]


def test_decode_rows_are_a_decode_step(orc):
    wl = _wl(vocab=300)
    ctx = np.array([5, 40, 17], np.int32)
    kv, layers = _state(wl, ctx, 1)
    x = synth.activations(np.random.default_rng(1), 3, wl.hidden)
    head = synth.head_weights(wl)
    kp, vp = _pools(kv)
    a, la = orc.mixed_stack(wl, layers, kp, vp, x, kv.pages.block_table, np.arange(3), ctx, head=head)
    kp, vp = _pools(kv)
    b, lb = orc.decode_stack(wl, layers, kp, vp, x, kv.pages.block_table, ctx, head=head)
    np.testing.assert_array_equal(a[-1], b[-1])
    np.testing.assert_array_equal(la, lb)


def test_runs_of_tokens_are_a_verification_step_in_any_row_order(orc):
    wl = _wl()
    ctx = np.array([5, 40, 17], np.int32)
    t = 4
    kv, layers = _state(wl, ctx, t)
    x = synth.activations(np.random.default_rng(2), 3 * t, wl.hidden)
    kp, vp = _pools(kv)
    want, _ = orc.verify_stack(wl, layers, kp, vp, x, kv.pages.block_table, ctx, t)
    seq = np.repeat(np.arange(3), t)
    pos = (ctx[:, None] + np.arange(t)[None, :]).reshape(-1)
    perm = np.random.default_rng(3).permutation(3 * t)
    kp, vp = _pools(kv)
    got, _ = orc.mixed_stack(wl, layers, kp, vp, x[perm], kv.pages.block_table, seq[perm], pos[perm])
    np.testing.assert_array_equal(got[-1], want[-1][perm])


def test_a_prompt_in_chunks_equals_the_prompt_at_once(orc):
    """Prefill of 20 tokens from an empty cache as one chunk, and as chunks of 8, 8 and 4
    (each chunk resuming where the last stopped), with a decode row of another sequence in
    every step: the same outputs for every prompt token."""
    wl = _wl()
    ctx = np.array([0, 33], np.int32)
    kv, layers = _state(wl, ctx, 20)
    x = synth.activations(np.random.default_rng(4), 20, wl.hidden)
    xd = synth.activations(np.random.default_rng(5), 3, wl.hidden)
    kp, vp = _pools(kv)
    whole, _ = orc.mixed_stack(wl, layers, kp, vp, x, kv.pages.block_table, np.zeros(20), np.arange(20))
    kp, vp = _pools(kv)
    pieces = []
    for step, (a, b) in enumerate([(0, 8), (8, 16), (16, 20)]):
        xs = np.concatenate([xd[step:step + 1], x[a:b]])
        seq = np.concatenate([[1], np.zeros(b - a, np.int64)])
        pos = np.concatenate([[33 + step], np.arange(a, b)])
        out, _ = orc.mixed_stack(wl, layers, kp, vp, xs, kv.pages.block_table, seq, pos)
        pieces.append(out[-1][1:])
    np.testing.assert_array_equal(np.concatenate(pieces), whole[-1])
