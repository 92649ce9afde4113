"""Pins of the oracle's speculative verification step (no GPU).

The verification step runs T tokens per sequence through the layer stack at once (Leone,
"What ships": exact speculative verification).  Its oracle goes layer by layer and, inside a
layer, token by token.  The pins tie that loop structure to plain decoding: with T = 1 it is a
decode step, T tokens equal T decode steps run one after another (a different loop order), no
token sees the tokens after it, and the acceptance rule has closed forms.
"""
import dataclasses

import numpy as np
import pytest

import synth


def _setup(t, kv_dtype=synth.KV_F16, n_layers=2, vocab=0, qk_norm=False):
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], n_layers=n_layers, batch=3, kv_dtype=kv_dtype, vocab=vocab,
                             qk_norm=qk_norm)
    ctx = np.array([5, 31, 16], np.int32)
    kv = synth.kv_state(wl, ctx, n_layers=n_layers, extra_slot=t)
    layers = [synth.layer_weights(wl, layer) for layer in range(n_layers)]
    x = synth.activations(np.random.default_rng(40 + t), 3 * t, wl.hidden)
    head = synth.head_weights(wl) if vocab else None
    return wl, ctx, kv, layers, x, head


def _pools(kv):
    return [p.copy() for p in kv.k_pools], [p.copy() for p in kv.v_pools]


def test_one_token_is_a_decode_step(orc):
    wl, ctx, kv, layers, x, head = _setup(1, vocab=300)
    kp, vp = _pools(kv)
    outs, logits = orc.verify_stack(wl, layers, kp, vp, x, kv.pages.block_table, ctx, 1, head=head)
    kp2, vp2 = _pools(kv)
    outs2, logits2 = orc.decode_stack(wl, layers, kp2, vp2, x, kv.pages.block_table, ctx, head=head)
    for a, b in zip(outs, outs2):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(logits, logits2)


@pytest.mark.parametrize("kv_dtype", [synth.KV_F16, synth.KV_Q8_0])
def test_t_tokens_equal_t_decode_steps(orc, kv_dtype):
    """Layer-outer (the verification step) against token-outer (T whole decode steps)."""
    t = 4
    wl, ctx, kv, layers, x, head = _setup(t, kv_dtype=kv_dtype, vocab=300, qk_norm=True)
    kp, vp = _pools(kv)
    outs, logits = orc.verify_stack(wl, layers, kp, vp, x, kv.pages.block_table, ctx, t, head=head)
    kp2, vp2 = _pools(kv)
    xs = x.reshape(3, t, -1)
    for j in range(t):
        o, lg = orc.decode_stack(wl, layers, kp2, vp2, xs[:, j], kv.pages.block_table, ctx + j, head=head)
        np.testing.assert_array_equal(outs[-1].reshape(3, t, -1)[:, j], o[-1])
        np.testing.assert_array_equal(logits.reshape(3, t, -1)[:, j], lg)
    for a, b in zip(kp + vp, kp2 + vp2):
        np.testing.assert_array_equal(a, b)


def test_tokens_do_not_see_later_tokens(orc):
    t = 3
    wl, ctx, kv, layers, x, _ = _setup(t)
    kp, vp = _pools(kv)
    outs, _ = orc.verify_stack(wl, layers, kp, vp, x, kv.pages.block_table, ctx, t)
    x2 = x.reshape(3, t, -1).copy()
    x2[:, t - 1] += 1.0
    kp2, vp2 = _pools(kv)
    outs2, _ = orc.verify_stack(wl, layers, kp2, vp2, x2.reshape(3 * t, -1), kv.pages.block_table, ctx, t)
    a, b = outs[-1].reshape(3, t, -1), outs2[-1].reshape(3, t, -1)
    np.testing.assert_array_equal(a[:, :t - 1], b[:, :t - 1])
    assert np.abs(a[:, t - 1] - b[:, t - 1]).max() > 1e-3


def test_acceptance_closed_forms(orc):
    draft = np.array([[7, 1, 2, 3], [7, 1, 2, 3], [7, 9, 2, 3], [7, 1, 2, 3], [5, 5, 5, 5]])
    sampled = np.array([[1, 2, 3, 4], [1, 2, 8, 4], [1, 2, 3, 4], [2, 2, 3, 4], [5, 5, 5, 5]])
    # all proposals match / the second mismatches / the first mismatches / none / row 4 all equal
    assert orc.spec_accept(sampled, draft).tolist() == [3, 2, 0, 0, 3]
    assert orc.spec_accept(np.array([[4]]), np.array([[9]])).tolist() == [0]
