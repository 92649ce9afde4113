"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

The pages print no worked values, so every pin is a closed form, an invariant, a
special case that reduces to a library routine, or a brute-force second
implementation (tests/refimpl.py) that shares no code with oracle.c.
"""
import json
import math
import os

import numpy as np
import pytest

import refimpl
import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "handpacked.json")


@pytest.fixture(scope="module")
def gold():
    with open(GOLD) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- fp16

def test_f16_decode_all_bit_patterns(orc):
    bits = np.arange(65536, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_f16_encode_matches_numpy(orc):
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000),
        # exact ties between neighbouring halves, normal and subnormal, and the overflow edge
        (np.arange(1, 200, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (1024 + np.arange(0, 300) + 0.5) * 2.0 ** -10,
        [65504.0, 65519.99, 65520.0, 65536.0, 1e6, -65520.0, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 0.0, -0.0],
    ])
    with np.errstate(over="ignore"):  # the overflow edge rounds to infinity on purpose
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.f64_to_f16(v) for v in vals], dtype=np.uint16)
    assert (got == want).all(), vals[got != want][:5]


# ----------------------------------------------------------------------------- Q4_K

def _q4k_expect(name):
    i = np.arange(256)
    j = i // 32
    if name == "q4k_a":
        return (j + 1) * (i % 16) - j
    if name == "q4k_b":
        return 0.25 * 63 * (15 - (i % 16)) - 0.125 * 63
    if name == "q4k_c":
        return 2.0 * (32 + j) * ((7 * i) % 16) - (63 - j)
    raise KeyError(name)


@pytest.mark.parametrize("name", ["q4k_a", "q4k_b", "q4k_c"])
def test_q4k_handpacked(orc, gold, name):
    e = gold[name]
    q = {"q4k_a": [i % 16 for i in range(256)], "q4k_b": [15 - (i % 16) for i in range(256)],
         "q4k_c": [(7 * i) % 16 for i in range(256)]}[name]
    assert refimpl.pack_q4k_block(e["d"], e["dmin"], e["sc"], e["m"], q).hex() == e["hex"]
    got = orc.dequant("q4k", np.frombuffer(bytes.fromhex(e["hex"]), np.uint8))
    np.testing.assert_array_equal(got, _q4k_expect(name))


def test_q4k_scale_packing_bijection():
    rng = np.random.default_rng(2)
    for _ in range(2000):
        s = bytes(rng.integers(0, 256, 12, dtype=np.uint8))
        sc, mn = refimpl.unpack_q4k_scales(s)
        assert refimpl.pack_q4k_scales(sc, mn) == s
    for j in range(8):  # each 6-bit field alone, every value
        for v in range(64):
            sc = [0] * 8
            mn = [0] * 8
            sc[j] = v
            assert refimpl.unpack_q4k_scales(refimpl.pack_q4k_scales(sc, mn)) == (sc, mn)
            sc[j], mn[j] = 0, v
            assert refimpl.unpack_q4k_scales(refimpl.pack_q4k_scales(sc, mn)) == (sc, mn)


def test_q4k_random_blocks_exact(orc):
    w = synth.q4k_weight(np.random.default_rng(3), 64, 1024)
    np.testing.assert_array_equal(orc.dequant("q4k", w), refimpl.decode_q4k(w).reshape(-1))


# ----------------------------------------------------------------------------- Q5_K

def _q5k_expect(name):
    i = np.arange(256)
    j = i // 32
    if name == "q5k_a":
        return (j + 1) * (i % 32) - j
    if name == "q5k_b":
        return 0.25 * 63 * (31 - (i % 32)) - 0.125 * 63
    if name == "q5k_c":
        return 2.0 * (32 + j) * ((7 * i) % 32) - (63 - j)
    raise KeyError(name)


@pytest.mark.parametrize("name", ["q5k_a", "q5k_b", "q5k_c"])
def test_q5k_handpacked(orc, gold, name):
    e = gold[name]
    q = {"q5k_a": [i % 32 for i in range(256)], "q5k_b": [31 - (i % 32) for i in range(256)],
         "q5k_c": [(7 * i) % 32 for i in range(256)]}[name]
    assert refimpl.pack_q5k_block(e["d"], e["dmin"], e["sc"], e["m"], q).hex() == e["hex"]
    got = orc.dequant("q5k", np.frombuffer(bytes.fromhex(e["hex"]), np.uint8))
    np.testing.assert_array_equal(got, _q5k_expect(name))


def test_q5k_random_blocks_exact(orc):
    w = synth.q5k_weight(np.random.default_rng(13), 64, 1024)
    np.testing.assert_array_equal(orc.dequant("q5k", w), refimpl.decode_q5k(w).reshape(-1))


def test_q5k_fifth_bits_one_at_a_time(orc):
    """Each high-bit byte bit, alone, adds 16 * d * sc to exactly one weight."""
    base = refimpl.pack_q5k_block(1.0, 0.0, [1] * 8, [0] * 8, [0] * 256)
    for l in (0, 7, 31):
        for bit in range(8):
            blk = bytearray(base)
            blk[16 + l] = 1 << bit
            got = orc.dequant("q5k", np.frombuffer(bytes(blk), np.uint8))
            want = np.zeros(256)
            want[64 * (bit // 2) + 32 * (bit % 2) + l] = 16.0
            np.testing.assert_array_equal(got, want)


# ----------------------------------------------------------------------------- Q6_K

def _q6k_expect(name):
    i = np.arange(256)
    if name == "q6k_a":
        return np.where((i // 16) % 2 == 0, 1, -1) * (i % 64 - 32)
    if name == "q6k_b":
        return np.where(i % 2 == 0, 0.0, 0.5 * -128 * 31)
    if name == "q6k_c":
        return 0.125 * ((i // 16) - 8) * ((5 * i + 3) % 64 - 32)
    raise KeyError(name)


@pytest.mark.parametrize("name", ["q6k_a", "q6k_b", "q6k_c"])
def test_q6k_handpacked(orc, gold, name):
    e = gold[name]
    q = {"q6k_a": [i % 64 for i in range(256)], "q6k_b": [32 if i % 2 == 0 else 63 for i in range(256)],
         "q6k_c": [(5 * i + 3) % 64 for i in range(256)]}[name]
    assert refimpl.pack_q6k_block(e["d"], e["scales"], q).hex() == e["hex"]
    got = orc.dequant("q6k", np.frombuffer(bytes.fromhex(e["hex"]), np.uint8))
    np.testing.assert_array_equal(got, _q6k_expect(name))


def test_q6k_random_blocks_exact(orc):
    w = synth.q6k_weight(np.random.default_rng(4), 48, 768)
    np.testing.assert_array_equal(orc.dequant("q6k", w), refimpl.decode_q6k(w).reshape(-1))


# ----------------------------------------------------------------------------- q8_0

def test_q8_0_handpacked(orc, gold):
    e = gold["q8_0_a"]
    got = orc.dequant("q8_0", np.frombuffer(bytes.fromhex(e["hex"]), np.uint8))
    codes = np.array(list(range(-127, 128)) + [0], dtype=np.float64)
    np.testing.assert_array_equal(got, 0.5 * codes)


def test_q8_0_quantizer_properties(orc):
    rng = np.random.default_rng(5)
    for trial in range(300):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        q, dbits = orc.q8_0_quantize_block(x)
        amax = np.max(np.abs(x))
        imax = int(np.argmax(np.abs(x)))
        assert abs(int(q[imax])) == 127 and np.sign(q[imax]) == np.sign(x[imax])
        d = float(np.float32(amax) / np.float32(127.0))
        assert dbits == int(np.array([d], np.float16).view(np.uint16)[0])
        # codes round x/d to nearest: |q*d - x| <= d/2 (with the unrounded d)
        assert np.all(np.abs(q.astype(np.float64) * d - x) <= d / 2 * (1 + 1e-6))
    q, dbits = orc.q8_0_quantize_block(np.zeros(32, np.float32))
    assert dbits == 0 and not q.any()


# ----------------------------------------------------------------------------- GEMM

@pytest.mark.parametrize("wtype", [synth.W_Q4_K, synth.W_Q6_K, synth.W_Q5_K, synth.W_Q8_0])
def test_gemm_matches_decoded_matmul(orc, wtype):
    rng = np.random.default_rng(6)
    n, k, b = 40, 768, 3
    w = synth.weight(rng, wtype, n, k)
    x = rng.standard_normal((b, k))
    got = orc.gemm(wtype, w, x, n, k)
    want = x @ refimpl.decode_matrix(wtype, w, n, k).T
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-9)
    # one-hot x selects column k0 of W exactly
    k0 = 517
    e = np.zeros((1, k))
    e[0, k0] = 1.0
    np.testing.assert_array_equal(orc.gemm(wtype, w, e, n, k)[0], refimpl.decode_matrix(wtype, w, n, k)[:, k0])


def test_gemm_brute_force_tiny(orc):
    w = synth.q4k_weight(np.random.default_rng(7), 1, 256)
    x = np.random.default_rng(8).standard_normal((1, 256))
    wd = refimpl.decode_q4k(w)[0]
    want = sum(float(wd[i]) * float(x[0, i]) for i in range(256))
    assert abs(orc.gemm(synth.W_Q4_K, w, x, 1, 256)[0, 0] - want) <= 1e-12 * max(1.0, abs(want))


def test_gemm_rejects_bad_k(orc):
    with pytest.raises(ValueError):
        orc.gemm(synth.W_Q4_K, np.zeros(144, np.uint8), np.zeros((1, 255)), 1, 255)


# ----------------------------------------------------------------------------- output head

@pytest.mark.parametrize("wtype,k", [(synth.W_Q6_K, 768), (synth.W_Q6_K, 512), (synth.W_Q4_K, 1024)])
def test_output_head_matches_brute_force(orc, wtype, k):
    """logits = W (rms(x) * g): numpy RMSNorm with the given eps and gain, then the decoded
    matrix (the final norm and output head of the Llama-3 shape; a 3-super-block Q6_K row is
    2-byte aligned)."""
    rng = np.random.default_rng(31)
    vocab, b = 50, 3
    w = synth.weight(rng, wtype, vocab, k)
    x = rng.standard_normal((b, k)) * np.array([[1.0], [1e-3], [40.0]])
    g = rng.uniform(0.5, 1.5, k).astype(np.float32)
    W = refimpl.decode_matrix(wtype, w, vocab, k)
    for eps in (1e-5, 0.7):  # a large eps makes a dropped or misplaced eps visible
        got = orc.output_head(x, g, eps, w, wtype, vocab)
        want = np.stack([refimpl.rms(x[i], g, eps) for i in range(b)]) @ W.T
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11 * np.abs(want).max())


def test_output_head_closed_forms(orc):
    """Constant rows: rms(c 1) = c / sqrt(c^2 + eps), so the logits are that factor times
    W g; a doubled gain doubles them; a row of zeros gives zeros for any eps > 0."""
    rng = np.random.default_rng(32)
    vocab, k = 24, 512
    w = synth.weight(rng, synth.W_Q6_K, vocab, k)
    W = refimpl.decode_matrix(synth.W_Q6_K, w, vocab, k)
    g = rng.uniform(0.5, 1.5, k).astype(np.float32)
    c, eps = 2.5, 0.3
    x = np.stack([np.full(k, c), np.zeros(k)])
    got = orc.output_head(x, g, eps, w, synth.W_Q6_K, vocab)
    np.testing.assert_allclose(got[0], c / math.sqrt(c * c + eps) * (W @ g.astype(np.float64)), rtol=1e-12)
    assert not got[1].any()
    got2 = orc.output_head(x[:1], (2 * g).astype(np.float32), eps, w, synth.W_Q6_K, vocab)
    np.testing.assert_allclose(got2[0], 2 * got[0], rtol=1e-14)


# ----------------------------------------------------------------------------- RMSNorm, RoPE, SiLU

def test_rmsnorm_closed_form_and_scale_invariance(orc):
    g = np.linspace(0.5, 1.5, 64).astype(np.float32)
    c, eps = 3.0, 1e-6
    got = orc.rmsnorm(np.full(64, c), g, eps)
    np.testing.assert_allclose(got, c / math.sqrt(c * c + eps) * g.astype(np.float64), rtol=1e-15)
    x = np.random.default_rng(9).standard_normal(64)
    a = orc.rmsnorm(x, g, 0.0)
    b = orc.rmsnorm(x * 7.5, g, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-14)
    np.testing.assert_allclose(np.mean((a / g) ** 2), 1.0, rtol=1e-13)


@pytest.mark.parametrize("style", [synth.ROPE_NEOX, synth.ROPE_NORM])
def test_rope_identities(orc, style):
    rng = np.random.default_rng(10)
    d, theta = 128, 5e5
    v = rng.standard_normal(d)
    np.testing.assert_array_equal(orc.rope(v, 0, theta, style), v)
    p = 12345
    r = orc.rope(v, p, theta, style)
    pairs = [(i, i + d // 2) if style == synth.ROPE_NEOX else (2 * i, 2 * i + 1) for i in range(d // 2)]
    for a, b in pairs:  # each pair keeps its norm
        assert abs(math.hypot(r[a], r[b]) - math.hypot(v[a], v[b])) < 1e-12
    np.testing.assert_allclose(orc.rope(r, -p, theta, style), v, atol=1e-12)
    for i in (0, 1, 17, 63):  # a unit vector on the first slot of pair i goes to (cos, sin)
        a, b = pairs[i]
        e = np.zeros(d)
        e[a] = 1.0
        out = orc.rope(e, p, theta, style)
        ang = p * theta ** (-2.0 * i / d)
        assert abs(out[a] - math.cos(ang)) < 1e-12 and abs(out[b] - math.sin(ang)) < 1e-12
        others = np.delete(out, [a, b])
        assert not others.any()


def test_silu_limits(orc):
    assert orc.silu(0.0) == 0.0
    assert abs(orc.silu(40.0) - 40.0) < 1e-12
    assert abs(orc.silu(-40.0)) < 1e-15
    assert abs(orc.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


# ----------------------------------------------------------------------------- attention

def _contig(rng, n, hkv, d):
    return rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))


def test_attention_brute_force_and_gqa(orc):
    rng = np.random.default_rng(11)
    n, hkv, d = 37, 3, 64
    K, V = _contig(rng, n, hkv, d)
    q = rng.standard_normal(d)
    for g in range(hkv):
        s = K[:, g] @ q / math.sqrt(d)
        w = np.exp(s - s.max())
        w /= w.sum()
        np.testing.assert_allclose(orc.attend_head(q, K, V, g), w @ V[:, g], rtol=1e-12, atol=1e-13)


def test_attention_special_cases(orc):
    rng = np.random.default_rng(12)
    hkv, d = 2, 64
    K, V = _contig(rng, 1, hkv, d)
    q = rng.standard_normal(d) * 100
    np.testing.assert_array_equal(orc.attend_head(q, K, V, 1), V[0, 1])  # one token: o = v exactly
    K, V = _contig(rng, 50, hkv, d)
    K[:] = K[0:1]  # identical keys: o = mean of V
    np.testing.assert_allclose(orc.attend_head(q, K, V, 0), V[:, 0].mean(axis=0), rtol=1e-12, atol=1e-14)
    V1 = np.ones_like(V)
    K, _ = _contig(rng, 50, hkv, d)
    np.testing.assert_allclose(orc.attend_head(q * 0.01, K, V1, 0), np.ones(d), rtol=1e-13)  # weights sum to 1


def test_lse_merge_of_page_aligned_splits(orc):
    rng = np.random.default_rng(13)
    n, hkv, d = 16 * 11 + 5, 2, 128
    K, V = _contig(rng, n, hkv, d)
    q = rng.standard_normal(d) * 3
    full = orc.attend_head(q, K, V, 1)
    for cuts in ([0, n], [0, 16, n], [0, 32, 96, 160, n], list(range(0, n, 16)) + [n]):
        parts = [orc.attend_partial(q, K, V, a, b, 1) for a, b in zip(cuts[:-1], cuts[1:])]
        o = orc.lse_merge(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]),
                          np.array([p[2] for p in parts]))
        np.testing.assert_allclose(o, full, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- pages

@pytest.mark.parametrize("kv_dtype", [synth.KV_F32, synth.KV_F16, synth.KV_Q8_0])
def test_gather_matches_page_decode_and_is_page_order_invariant(orc, kv_dtype):
    wl = synth.WORKLOADS["tiny"]
    import dataclasses
    wl = dataclasses.replace(wl, kv_dtype=kv_dtype, batch=3)
    ctx = np.array([1, 40, 16], dtype=np.int32)
    kv = synth.kv_state(wl, ctx, extra_slot=False)
    bt = kv.pages.block_table
    for is_v, pool in ((False, kv.k_pools[0]), (True, kv.v_pools[0])):
        got = orc.gather_kv(pool, kv_dtype, is_v, wl.n_kv_heads, wl.head_dim, bt, ctx)
        want = np.concatenate([refimpl.gather_row(pool, kv_dtype, is_v, wl.n_kv_heads, wl.head_dim, bt[b], ctx[b])
                               for b in range(3)])
        np.testing.assert_array_equal(got, want)
        assert np.isfinite(got).all()
        # move every page to a new physical slot: the logical gather is unchanged
        perm = np.random.default_rng(14).permutation(pool.shape[0])
        moved = np.empty_like(pool)
        moved[perm] = pool
        bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
        np.testing.assert_array_equal(orc.gather_kv(moved, kv_dtype, is_v, wl.n_kv_heads, wl.head_dim, bt2, ctx),
                                      got)


@pytest.mark.parametrize("kv_dtype", [synth.KV_F32, synth.KV_F16, synth.KV_Q8_0])
def test_append_stores_rounded_value(orc, kv_dtype):
    hkv, d = 2, 64
    hb = orc.head_bytes(kv_dtype, d)
    assert hb == refimpl.head_bytes(kv_dtype, d)
    pool = np.zeros((3, hkv * hb), np.uint8)
    bt = np.array([2, 0], np.int32)
    vec = np.random.default_rng(15).standard_normal(hkv * d) * 3
    for is_v in (False, True):
        orc.kv_append(pool, kv_dtype, is_v, hkv, d, bt, 21, vec)
        got = orc.gather_kv(pool, kv_dtype, is_v, hkv, d, bt[None], np.array([22]))[21]
        np.testing.assert_array_equal(got.reshape(-1), refimpl.store_round(vec, kv_dtype))
        pool[:] = 0


# ----------------------------------------------------------------------------- layer

def _tiny_layer_inputs(kv_dtype=None, qk_norm=None, batch=None, ctx=None, style=None):
    import dataclasses
    wl = synth.WORKLOADS["tiny"]
    rep = {}
    if kv_dtype is not None:
        rep["kv_dtype"] = kv_dtype
    if qk_norm is not None:
        rep["qk_norm"] = qk_norm
    if batch is not None:
        rep["batch"] = batch
    if style is not None:
        rep["rope_style"] = style
    wl = dataclasses.replace(wl, **rep)
    lw = synth.layer_weights(wl, 0)
    c = synth.ctx_lens(wl) if ctx is None else np.asarray(ctx, np.int32)
    kv = synth.kv_state(wl, c)
    x = synth.input_x(wl, len(c))
    return wl, lw, kv, x, c


@pytest.mark.parametrize("variant", [dict(), dict(qk_norm=True), dict(kv_dtype=synth.KV_F16, style=synth.ROPE_NORM),
                                     dict(kv_dtype=synth.KV_Q8_0, qk_norm=True)])
def test_layer_matches_numpy_brute_force(orc, variant):
    wl, lw, kv, x, c = _tiny_layer_inputs(batch=3, ctx=[128, 0, 33], **variant)
    kp, vp = kv.k_pools[0].copy(), kv.v_pools[0].copy()
    want = refimpl.brute_layer(wl, lw, kv.k_pools[0], kv.v_pools[0], x, kv.pages.block_table, c)
    got = orc.decode_layer(wl, lw, kp, vp, x, kv.pages.block_table, c)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-9 * np.abs(want).max())


def test_layer_batched_equals_rows_alone(orc):
    wl, lw, kv, x, c = _tiny_layer_inputs(batch=3, ctx=[5, 100, 47], qk_norm=True)
    bt = kv.pages.block_table
    kp, vp = kv.k_pools[0].copy(), kv.v_pools[0].copy()
    batched = orc.decode_layer(wl, lw, kp, vp, x, bt, c)
    for b in range(3):
        kp1, vp1 = kv.k_pools[0].copy(), kv.v_pools[0].copy()
        one = orc.decode_layer(wl, lw, kp1, vp1, x[b:b + 1], bt[b:b + 1], c[b:b + 1])
        np.testing.assert_array_equal(one[0], batched[b])
    # rows leaving or joining between steps: any subset in any order gives the same rows
    sub = [2, 0]
    kp2, vp2 = kv.k_pools[0].copy(), kv.v_pools[0].copy()
    part = orc.decode_layer(wl, lw, kp2, vp2, x[sub], bt[sub], c[sub])
    np.testing.assert_array_equal(part, batched[sub])


def test_layer_writes_new_token_at_position(orc):
    wl, lw, kv, x, c = _tiny_layer_inputs(batch=1, ctx=[37])
    kp, vp = kv.k_pools[0].copy(), kv.v_pools[0].copy()
    _, taps = orc.decode_layer(wl, lw, kp, vp, x, kv.pages.block_table, c, taps=True)
    got_k = orc.gather_kv(kp, wl.kv_dtype, False, wl.n_kv_heads, wl.head_dim, kv.pages.block_table, np.array([38]))
    np.testing.assert_array_equal(got_k[37].reshape(-1), refimpl.store_round(taps["k"][0], wl.kv_dtype))
    before = orc.gather_kv(kv.k_pools[0], wl.kv_dtype, False, wl.n_kv_heads, wl.head_dim, kv.pages.block_table,
                           np.array([37]))
    np.testing.assert_array_equal(got_k[:37], before)  # earlier tokens untouched
